"""palu_decode_attn_noalloc, the decode entry point that allocates nothing
(it works in the library's static per-GPU scratch), against palu_decode_attn
with a caller-owned workspace: bit-identical outputs on two calls in a row,
the second with a smaller input (the scratch keeps the first call's contents,
which must not leak into the second), in both key modes and with the value
latents returned; then once more with the ordinary entry point in between."""
import numpy as np
import pytest

import workloads as W
from tests.parity_util import dev

pytestmark = pytest.mark.gpu


def _call_both(cfg, mode, latent_out=False):
    import torch
    import rank_compressed_kv_amd as P
    t = W.generate(cfg)
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, mode=mode, rope_theta=theta,
                       latent_out=latent_out)
    q, hk, hv, bk, bv, lens = (dev(t[k]) for k in ("q", "h_k", "h_v", "b_k", "b_v", "lens"))
    width = cfg.rank if latent_out else cfg.head_dim
    shape = (cfg.batch, cfg.n_q_heads, width)
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    want = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, want, ws)
    P.palu_decode_attn_noalloc(desc, q, hk, hv, bk, bv, lens, got)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("mode", ["absorbed", "reconstruct"])
def test_noalloc_matches_workspace_call_twice(mode):
    import torch
    big = W.CONFIGS[3].scaled(batch=4, max_ctx=3000, ragged=(1, 3000), seed=210)
    small = W.CONFIGS[3].scaled(batch=2, max_ctx=700, ragged=(1, 700), seed=211)
    for i, cfg in enumerate((big, small)):
        print(f"[noalloc] {mode} call {i} B={cfg.batch} L={cfg.max_ctx}", flush=True)
        got, want = _call_both(cfg, mode)
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), f"{mode} call {i}"


def test_noalloc_latent_out_and_interleaved_calls():
    import torch
    cfg = W.CONFIGS[5].scaled(batch=3, max_ctx=1500, ragged=(1, 1500), seed=212)
    print("[noalloc] latent_out J-LRD", flush=True)
    got, want = _call_both(cfg, "reconstruct", latent_out=True)
    assert torch.equal(got, want)
    cfg = W.CONFIGS[3].scaled(batch=1, max_ctx=300, seed=213)
    got, want = _call_both(cfg, "absorbed")
    assert torch.equal(got, want)
