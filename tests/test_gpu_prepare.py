"""The prepare step: the query-side operands formed by palu_decode_attn_prepare
on a second stream (overlapping a cache write on the first), then a call with
prepared = 1, give exactly the outputs of the ordinary call, in every mode and
for the quantised caches."""
import numpy as np
import pytest

import workloads as W
from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache
from tests.parity_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["absorbed", "reconstruct", "full_rank", "int8", "int4"])
def test_prepared_call_is_the_same_call(kind):
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=1504)
    t = W.generate(cfg, parts=("decode", "append", "full", "i8", "i4"))
    q, lens = dev(t["q"]), dev(t["lens"])
    bk, bv = dev(t["b_k"]), dev(t["b_v"])
    mode = kind if kind in ("absorbed", "reconstruct", "full_rank") else "absorbed"
    G, r = cfg.n_groups, cfg.rank
    if kind == "full_rank":
        G, r = cfg.n_kv_heads, cfg.head_dim
    kw = dict(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
              head_dim=cfg.head_dim, n_groups=G, rank=r, max_ctx=cfg.max_ctx,
              dtype=P.PALU_BF16, mode=mode,
              rope_theta=cfg.rope_theta if mode == "reconstruct" else 0.0)
    plain, prep = P.attn_desc(**kw), P.attn_desc(**kw, prepared=True)
    if kind in ("int8", "int4"):
        pack = pack_i8_cache if kind == "int8" else pack_i4_cache
        b = kind[-1]
        sfx = "" if b == "8" else "_i4"
        cache = [dev(pack(t[f"k_i{b}"], "k")), dev(pack(t[f"v_i{b}"], "v")),
                 dev(t["sk" + sfx]), dev(t["sv" + sfx])]
        fn = P.palu_decode_attn_i8 if kind == "int8" else P.palu_decode_attn_i4
        call = lambda d, ws, out, s: fn(d, q, *cache, bk, bv, lens, out, ws, s)
    elif kind == "full_rank":
        k, v = dev(t["k_full"]), dev(t["v_full"])
        call = lambda d, ws, out, s: P.palu_decode_attn(d, q, k, v, None, None, lens, out, ws, s)
    else:
        hk, hv = dev(t["h_k"]), dev(t["h_v"])
        call = lambda d, ws, out, s: P.palu_decode_attn(d, q, hk, hv, bk, bv, lens, out, ws, s)
    nws = P.palu_decode_attn_workspace(plain)
    ws1 = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out1 = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out1)
    main = torch.cuda.current_stream()
    call(plain, ws1, out1, main)
    # a cache write on the main stream while the prepare step runs on a side stream
    adesc = P.append_desc(batch=cfg.batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                          rank=cfg.rank, max_ctx=cfg.max_ctx, dtype=P.PALU_BF16)
    spare_k, spare_v = dev(t["h_k"]), dev(t["h_v"])
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        P.palu_decode_attn_prepare(prep, q, None if kind == "full_rank" else bk, ws2, side)
    P.latent_append(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), spare_k, spare_v, dev(t["pos"]))
    main.wait_stream(side)
    call(prep, ws2, out2, main)
    torch.cuda.synchronize()
    assert torch.isfinite(out1).all()
    assert torch.equal(out1, out2), kind


@pytest.mark.parametrize("rank", [256, 128])
def test_reconstruct_prepare_once_serves_later_calls(rank):
    """In RECONSTRUCT mode the prepared operand is B_k transposed alone: one
    palu_decode_attn_prepare serves every later prepared call with the same
    b_k and workspace (new queries and caches each call), each output equal to
    the ordinary call's."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=1504, rank=rank)
    base = W.generate(cfg)
    bk, bv = dev(base["b_k"]), dev(base["b_v"])
    kw = dict(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
              head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank, max_ctx=cfg.max_ctx,
              dtype=P.PALU_BF16, mode="reconstruct", rope_theta=cfg.rope_theta)
    plain, prep = P.attn_desc(**kw), P.attn_desc(**kw, prepared=True)
    nws = P.palu_decode_attn_workspace(plain)
    ws1 = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nws, dtype=torch.uint8, device="cuda")
    P.palu_decode_attn_prepare(prep, dev(base["q"]), bk, ws2)
    for call in range(3):
        t = W.generate(cfg, seed=900 + call)
        q, hk, hv, lens = dev(t["q"]), dev(t["h_k"]), dev(t["h_v"]), dev(t["lens"])
        out1 = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32,
                           device="cuda")
        out2 = torch.empty_like(out1)
        P.palu_decode_attn(plain, q, hk, hv, bk, bv, lens, out1, ws1)
        P.palu_decode_attn(prep, q, hk, hv, bk, bv, lens, out2, ws2)
        torch.cuda.synchronize()
        assert torch.isfinite(out1).all()
        assert torch.equal(out1, out2), (rank, call)
