"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs, element by element, at sizes the oracle finishes in
seconds; the bar is max |d| <= 2e-2 and relative L2 <= 5e-3 (fp32 workloads:
1e-4 and 1e-5)."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from tests.parity_util import assert_close, dev, run_decode

pytestmark = pytest.mark.gpu

# reduced context so the oracle is quick; lengths chosen off the 64-token grid
SMALL = {
    1: W.CONFIGS[1],
    2: W.CONFIGS[2].scaled(batch=2, max_ctx=1000),
    3: W.CONFIGS[3].scaled(batch=2, max_ctx=1500),
    4: W.CONFIGS[4].scaled(max_ctx=3000),
    5: W.CONFIGS[5].scaled(batch=4, max_ctx=2048, ragged=(1, 2048)),
}
CASES = [(i, m) for i in SMALL for m in SMALL[i].modes]


def _tol(cfg):
    return dict(max_abs=1e-4, rel_l2=1e-5) if cfg.dtype == "f32" else {}


def _oracle(cfg, t, theta, lens=None):
    lens = t["lens"] if lens is None else lens
    return O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], lens,
                              rope_theta=theta)


@pytest.mark.parametrize("idx,mode", CASES)
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_parity_reduced(idx, mode, split_tokens):
    cfg = SMALL[idx]
    t = W.generate(cfg)
    print(f"[parity] cfg{idx} {cfg.name} mode={mode} split={split_tokens} lens={t['lens'].tolist()}",
          flush=True)
    got, theta = run_decode(cfg, t, mode, split_tokens=split_tokens)
    want = _oracle(cfg, t, theta)
    assert_close(got, want, what=f"cfg{idx}/{mode}", **_tol(cfg))


@pytest.mark.parametrize("idx", [2, 4, 5])
@pytest.mark.parametrize("split_tokens", [0, 64, 192])
def test_parity_absorbed_other_shapes(idx, split_tokens):
    """Absorbed keys (no RoPE) on the other head layouts: 4 query heads per group
    (MHA), rank 128 with outlier channels, and one 32-head group at rank 512."""
    cfg = SMALL[idx]
    t = W.generate(cfg)
    print(f"[absorbed] cfg{idx} split={split_tokens}", flush=True)
    got, theta = run_decode(cfg, t, "absorbed", split_tokens=split_tokens)
    assert theta == 0.0
    assert_close(got, _oracle(cfg, t, 0.0), what=f"absorbed cfg{idx}")


@pytest.mark.parametrize("idx", [1, 3])
def test_reconstruct_without_rope_equals_absorbed(idx):
    """With theta = 0 the two key paths compute the same scores."""
    cfg = SMALL[idx]
    t = W.generate(cfg)
    a, _ = run_decode(cfg, t, "absorbed")
    b, _ = run_decode(cfg, t, "reconstruct", rope_theta=0.0)
    assert_close(a, b, what="absorbed vs reconstruct", **_tol(cfg))


@pytest.mark.parametrize("idx,mode", [(1, "absorbed"), (1, "reconstruct"), (3, "absorbed"),
                                      (3, "reconstruct"), (5, "reconstruct")])
def test_length_edges_and_poisoned_tail(idx, mode):
    """Lengths 0, 1, around the split size and the capacity; rows past each length
    are NaN, so any read beyond the context shows up."""
    base = SMALL[idx]
    L = 640
    edge = [0, 1, 63, 64, 65, 129, 511, L]
    cfg = base.scaled(batch=len(edge), max_ctx=L, ragged=None)
    t = W.generate(cfg, lens=np.array(edge))
    hk, hv = W.poison_tail(t["h_k"], t["lens"]), W.poison_tail(t["h_v"], t["lens"])
    for st in (64, 128, 0):
        print(f"[edges] cfg{idx} mode={mode} split={st}", flush=True)
        got, theta = run_decode(cfg, t, mode, split_tokens=st, h_k=hk, h_v=hv)
        want = _oracle(cfg, t, theta)
        assert np.all(got[0] == 0.0)
        assert_close(got, want, what=f"edges cfg{idx}/{mode}/split{st}", **_tol(cfg))


def bump_keys(hk, up, down):
    """Key latents (bf16 bits) of tokens `up` times 16 and of tokens `down`
    times -16: exponent + 4 (no overflow at these magnitudes), sign flipped."""
    hk = hk.copy()
    for rows, sign in ((up, 0), (down, 0x8000)):
        f = hk[:, :, rows, :].astype(np.uint32)
        f = np.where((f & 0x7F80) != 0, f + (4 << 7), f) ^ sign
        hk[:, :, rows, :] = f.astype(np.uint16)
    return hk


@pytest.mark.parametrize("idx", [2, 3, 5])
def test_reconstruct_rescale_inside_tile_pair(idx):
    """The rank-256 kernels take a pair of 16-token tiles' values in one MFMA,
    the first tile's weights waiting for the second: tokens of second tiles
    (16..31 of each 32) whose key latents are scaled by 16 and by -16 (exact in
    bf16) raise the running max by far more than the lazy-rescale threshold, so
    the kept weights are rescaled too; lengths leave odd and even tile counts.
    At rank 512 (four waves per KV head, each with a quarter of the columns)
    the same jumps check that the four waves, which add the partial scores in
    one order, take the same rescale decisions."""
    cfg = SMALL[idx].scaled(batch=3, max_ctx=420, ragged=None)
    t = W.generate(cfg, lens=np.array([420, 405, 37]))
    t = dict(t, h_k=bump_keys(t["h_k"], [17, 18, 19, 150, 389, 28], [20, 21, 22, 152, 400, 30]))
    for st in (0, 64, 128):
        print(f"[pair-rescale] cfg{idx} split={st}", flush=True)
        got, theta = run_decode(cfg, t, "reconstruct", split_tokens=st)
        assert_close(got, _oracle(cfg, t, theta), what=f"pair rescale cfg{idx} split={st}")


# (KV heads per group s, rank r): the granularities at 75% key compression
# (M-LRD s=1 r=32 ... J-LRD s=8 r=256) and rank 512 with 2, 4 and 8 heads
GROUPINGS = [(1, 32), (2, 64), (4, 128), (8, 256), (1, 128), (2, 256), (2, 512), (4, 512),
             (8, 512), (1, 64), (2, 32), (2, 128)]


@pytest.mark.parametrize("s,r", GROUPINGS)
def test_reconstruct_head_groupings(s, r):
    """Rebuilt and rotated keys for every head grouping the MFMA kernel serves:
    one, two or four KV heads per workgroup, and groups whose heads are spread
    over several workgroups of the same context split."""
    cfg = W.CONFIGS[3].scaled(n_groups=8 // s, rank=r, batch=2, max_ctx=700, seed=40 + s)
    t = W.generate(cfg)
    print(f"[grouping] s={s} r={r}", flush=True)
    for st in (0, 128):
        got, theta = run_decode(cfg, t, "reconstruct", split_tokens=st)
        assert theta > 0
        assert_close(got, _oracle(cfg, t, theta), what=f"s={s} r={r} split={st}")


@pytest.mark.parametrize("s,r,hq", [(1, 32, 8), (2, 64, 16), (1, 64, 24)])
def test_reconstruct_groups_in_one_workgroup(s, r, hq):
    """Groups of one or two KV heads whose four consecutive KV heads share a
    workgroup (each group's tile in its own LDS ring), with one, two and
    three query heads per KV head, ragged lengths (one of them 0) and a
    NaN-poisoned tail."""
    cfg = W.CONFIGS[3].scaled(n_groups=8 // s, rank=r, batch=4, max_ctx=530, n_q_heads=hq,
                              seed=70 + s)
    t = W.generate(cfg, lens=np.array([530, 301, 0, 17]))
    hk, hv = W.poison_tail(t["h_k"], t["lens"]), W.poison_tail(t["h_v"], t["lens"])
    print(f"[groups] s={s} r={r} hq={hq}", flush=True)
    for st in (0, 64):
        got, theta = run_decode(cfg, t, "reconstruct", split_tokens=st, h_k=hk, h_v=hv)
        assert theta > 0
        assert_close(got, _oracle(cfg, t, theta), what=f"groups s={s} r={r} hq={hq} split={st}")


@pytest.mark.parametrize("hq,r", [(24, 128), (40, 256), (64, 64), (32, 256)])
def test_absorbed_many_query_heads_per_group(hq, r):
    """Absorbed keys with more than 16 query heads a group (two head blocks a
    workgroup): 24 heads (a partial second block), 40 (a second slice whose
    second block is empty), 64 (two full slices), 32; ragged lengths (one
    0), a NaN-poisoned tail and several split sizes."""
    cfg = W.CONFIGS[3].scaled(n_q_heads=hq, n_kv_heads=8, n_groups=1, rank=r, batch=3,
                              max_ctx=600, seed=80 + hq)
    t = W.generate(cfg, lens=np.array([600, 0, 233]))
    hk, hv = W.poison_tail(t["h_k"], t["lens"]), W.poison_tail(t["h_v"], t["lens"])
    print(f"[many-heads] hq={hq} r={r}", flush=True)
    for st in (0, 64, 192):
        got, _ = run_decode(cfg, t, "absorbed", split_tokens=st, h_k=hk, h_v=hv)
        assert np.all(got[1] == 0.0)
        assert_close(got, _oracle(cfg, t, 0.0), what=f"absorbed hq={hq} r={r} split={st}")


@pytest.mark.parametrize("s,r", [(1, 32), (2, 64), (4, 128), (8, 256)])
def test_absorbed_head_groupings(s, r):
    """Absorbed keys for every head grouping at 75% compression: ranks 32-256 on
    the MFMA kernel, and 32 query heads per group (two head slices that share
    the latent tiles)."""
    cfg = W.CONFIGS[3].scaled(n_groups=8 // s, rank=r, batch=2, max_ctx=700, seed=50 + s)
    t = W.generate(cfg)
    for st in (0, 128):
        got, theta = run_decode(cfg, t, "absorbed", split_tokens=st)
        assert_close(got, _oracle(cfg, t, 0.0), what=f"absorbed s={s} r={r} split={st}")


@pytest.mark.parametrize("mode", ["absorbed", "reconstruct"])
def test_more_than_64_splits(mode):
    """79 splits of 64 tokens: the merge that stages split states through LDS
    (the fast merge keeps at most 64 split states in one wave)."""
    cfg = W.CONFIGS[4].scaled(max_ctx=5000)
    t = W.generate(cfg)
    print(f"[many splits] cfg4 mode={mode}", flush=True)
    got, theta = run_decode(cfg, t, mode, split_tokens=64)
    assert_close(got, _oracle(cfg, t, theta), what=f"79 splits/{mode}")


def _run_full(cfg, t, split_tokens=0, lens=None):
    import torch
    import rank_compressed_kv_amd as P
    ln = dev(t["lens"] if lens is None else lens)
    out = P.full_rank_attention(dev(t["q"]), dev(t["k_full"]), dev(t["v_full"]), ln,
                                split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("idx", [2, 3, 5])
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_full_rank_baseline(idx, split_tokens):
    """The uncompressed baseline (full bf16 K and V, keys cached rotated) on the
    MHA, GQA and ragged shapes: ordinary decode attention."""
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "full"))
    print(f"[full rank] cfg{idx} split={split_tokens}", flush=True)
    got = _run_full(cfg, t, split_tokens)
    want = O.full_rank_attention(t["q"], t["k_full"], t["v_full"], t["lens"])
    assert_close(got, want, what=f"full rank cfg{idx}")


def test_full_rank_length_edges():
    cfg = SMALL[3].scaled(batch=8, max_ctx=640, ragged=None)
    edge = np.array([0, 1, 63, 64, 65, 129, 511, 640])
    t = W.generate(cfg, parts=("decode", "full"), lens=edge)
    for st in (64, 0):
        got = _run_full(cfg, t, st)
        assert np.all(got[0] == 0.0)
        want = O.full_rank_attention(t["q"], t["k_full"], t["v_full"], edge)
        assert_close(got, want, what=f"full rank edges split={st}")


@pytest.mark.parametrize("idx,mode", [(3, "absorbed"), (3, "reconstruct"), (2, "reconstruct"),
                                      (5, "reconstruct"), (4, "absorbed")])
def test_latent_output_without_bv(idx, mode):
    """latent_out: the call returns the weighted value latents u* [B, Hq, r] and
    never reads B_v (passed as None), for the caller to fuse B_v with W_o."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = SMALL[idx]
    t = W.generate(cfg)
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    print(f"[latent out] cfg{idx} mode={mode}", flush=True)
    for st in (0, 64):
        got = P.decode_attention(dev(t["q"]), dev(t["h_k"]), dev(t["h_v"]), dev(t["b_k"]), None,
                                 dev(t["lens"]), n_kv_heads=cfg.n_kv_heads, mode=mode,
                                 rope_theta=theta, split_tokens=st, latent_out=True)
        torch.cuda.synchronize()
        want = O.decode_value_latents(t["q"], t["h_k"], t["h_v"], t["b_k"], t["lens"],
                                      cfg.group_dim, rope_theta=theta)
        assert got.shape == (cfg.batch, cfg.n_q_heads, cfg.rank)
        assert_close(got.cpu().numpy().astype(np.float64), want, what=f"u* cfg{idx}/{mode}")


def test_null_lens_means_full_capacity():
    cfg = SMALL[3].scaled(max_ctx=300)
    t = W.generate(cfg)
    got, theta = run_decode(cfg, t, "reconstruct", lens=False)
    want = _oracle(cfg, t, theta, lens=np.full(cfg.batch, cfg.max_ctx))
    assert_close(got, want, what="lens=NULL")


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_latent_append(idx):
    """h[b, g, pos[b]] = x[b] A: bf16 rows agree with the oracle's fp32-then-bf16
    rounding except where the exact value sits within the fp32 summation error
    of a rounding midpoint; rows other than pos[b] are untouched."""
    base = W.CONFIGS[idx]
    _check_append(base.scaled(batch=min(base.batch, 4), max_ctx=64, ragged=None), 0)


# the transposed projection (one-pass kernel): every config, a batch that
# takes two passes of 8 sequences, and d_model 3072 (a partial 2048-chunk slab)
APPEND_COLS = {f"cfg{i}": W.CONFIGS[i].scaled(batch=min(W.CONFIGS[i].batch, 4), max_ctx=64,
                                              ragged=None) for i in (1, 2, 3, 4, 5)}
APPEND_COLS["b11"] = W.CONFIGS[3].scaled(batch=11, max_ctx=32, ragged=None, seed=61)
APPEND_COLS["dm3072"] = W.CONFIGS[2].scaled(batch=3, max_ctx=32, ragged=None, n_q_heads=24,
                                            n_kv_heads=24, n_groups=6, seed=62)


@pytest.mark.parametrize("name", sorted(APPEND_COLS))
def test_latent_append_transposed_projection(name):
    """The same write from a_k, a_v stored [G*r, d_model] (PALU_A_OUT_IN)."""
    _check_append(APPEND_COLS[name], 1)


def _check_append(cfg, a_layout):
    import torch
    import rank_compressed_kv_amd as P
    t = W.generate(cfg, parts=("decode", "append"))
    print(f"[append] B={cfg.batch} d_model={cfg.d_model} G={cfg.n_groups} r={cfg.rank} "
          f"a_layout={a_layout}", flush=True)
    hk, hv = dev(t["h_k"]), dev(t["h_v"])
    before_k = hk.clone()
    ak, av = t["a_k"], t["a_v"]
    if a_layout:
        ak, av = np.ascontiguousarray(ak.T), np.ascontiguousarray(av.T)
    P.latent_append(dev(t["x"]), dev(ak), dev(av), hk, hv, dev(t["pos"]), a_layout=a_layout)
    torch.cuda.synchronize()
    G, r = cfg.n_groups, cfg.rank
    for name, cache, a in (("k", hk, t["a_k"]), ("v", hv, t["a_v"])):
        want64 = O.latent_project(t["x"], a)                  # [B, G*r]
        c = cache.cpu()
        for b, pos in enumerate(t["pos"]):
            row = c[b, :, int(pos), :].reshape(-1)
            if cfg.dtype == "bf16":
                got_bits = row.view(torch.int16).numpy().view(np.uint16)
                want_bits = O.append_rows_bf16(want64[b])
                bad = got_bits != want_bits
                if bad.any():
                    # the GPU's fp32 sum S lies within E = d_model * 2^-24 *
                    # sum |x_i a_i| of the exact value (any summation order), and
                    # it stores bf16(S); rounding is monotone, so the stored
                    # value must lie between the roundings of exact - E and
                    # exact + E (several bf16 steps apart where the sum cancels)
                    E = (np.sum(np.abs(O.to_f64(t["x"][b])[:, None] * O.to_f64(a)), 0)
                         * cfg.d_model * 2.0 ** -24)
                    val = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
                    lo = val(O.append_rows_bf16(want64[b] - E))
                    hi = val(O.append_rows_bf16(want64[b] + E))
                    g = val(got_bits)
                    assert np.all((g >= lo) & (g <= hi)), name
                assert bad.mean() < 0.01
            else:
                np.testing.assert_allclose(row.numpy(), want64[b], rtol=1e-5, atol=1e-5)
    # untouched rows
    mask = torch.ones(cfg.batch, cfg.max_ctx, dtype=torch.bool)
    for b, pos in enumerate(t["pos"]):
        mask[b, int(pos)] = False
    assert torch.equal(hk.cpu()[:, :, :, :].permute(0, 2, 1, 3)[mask],
                       before_k.cpu().permute(0, 2, 1, 3)[mask])


def test_append_workspace_reuse():
    """The arrival counters return to zero after every call, so one workspace
    serves call after call (batch sizes and positions changing) with results
    bit-identical to calls on a fresh workspace."""
    import torch
    import rank_compressed_kv_amd as P
    ws = None
    for i, batch in enumerate((4, 2, 4)):
        cfg = W.CONFIGS[3].scaled(batch=batch, max_ctx=16, seed=100 + i)
        t = W.generate(cfg, parts=("decode", "append"))
        x, ak, av, pos = dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), dev(t["pos"])
        hk, hv = dev(t["h_k"]), dev(t["h_v"])
        hk2, hv2 = hk.clone(), hv.clone()
        desc = P.append_desc(batch=batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                             rank=cfg.rank, max_ctx=16, dtype=P.PALU_BF16)
        if ws is None:
            ws = torch.zeros(P.palu_latent_append_workspace(desc), dtype=torch.uint8,
                             device="cuda")
        P.palu_latent_append(desc, x, ak, av, hk, hv, pos, ws)
        P.latent_append(x, ak, av, hk2, hv2, pos)          # fresh zeroed workspace
        torch.cuda.synchronize()
        assert torch.equal(hk, hk2) and torch.equal(hv, hv2)
        assert int(ws[:256].count_nonzero()) == 0


@pytest.mark.parametrize("a_layout", [0, 1])
def test_append_out_of_range_rows_skipped(a_layout):
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=16)
    t = W.generate(cfg, parts=("decode", "append"))
    hk, hv = dev(t["h_k"]), dev(t["h_v"])
    before = (hk.clone(), hv.clone())
    pos = torch.tensor([-1, 16], dtype=torch.int32, device="cuda")
    ak, av = dev(t["a_k"]), dev(t["a_v"])
    if a_layout:
        ak, av = ak.t().contiguous(), av.t().contiguous()
    P.latent_append(dev(t["x"]), ak, av, hk, hv, pos, a_layout=a_layout)
    torch.cuda.synchronize()
    assert torch.equal(hk, before[0]) and torch.equal(hv, before[1])
