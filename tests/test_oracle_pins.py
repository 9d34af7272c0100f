"""Pins of the CPU oracle to things other than itself.

Each test ties the oracle to a closed form, a library routine, brute force on
tiny inputs or an identity the pages state, so that a dropped term, a wrong
sign, a wrong index or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import palu_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _arr(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------- goldens ---

def test_golden_quantize_rows_i8(golden):
    """Hand-derived codes: amax 2 gives inv 63.5; -63.5 and 0.5 are ties and go
    to the even neighbour; a zero row has scale 0."""
    c = golden["quantize_rows_i8"]
    codes, scales = O.quantize_rows_i8(np.array(c["h"], dtype=np.float32))
    np.testing.assert_array_equal(codes, np.array(c["codes"], dtype=np.int8))
    np.testing.assert_allclose(scales * 127.0, c["scales_times_127"], rtol=1e-7, atol=0)


def test_golden_two_token_softmax(golden):
    c = golden["two_token_softmax"]
    out = O.decode_attention(_arr(c["q"]), _arr(c["h_k"]), _arr(c["h_v"]), _arr(c["b_k"]),
                             _arr(c["b_v"]), np.array(c["lens"]), rope_theta=c["rope_theta"])
    np.testing.assert_allclose(out, _arr(c["out"]), rtol=0, atol=1e-12)


def test_golden_project_then_reconstruct(golden):
    c = golden["project_then_reconstruct"]
    h = O.latent_project(_arr(c["x"]), _arr(c["a"]))
    np.testing.assert_array_equal(h, _arr(c["h"]))
    np.testing.assert_array_equal(O.reconstruct(h, _arr(c["b"])), _arr(c["y"]))


def test_golden_rope_quarter_turn(golden):
    c = golden["rope_quarter_turn"]
    keys = np.tile(_arr(c["key"]), (len(c["positions"]), 1))
    rot = O.apply_rope(keys, np.array(c["positions"]), c["theta"])
    np.testing.assert_allclose(rot, _arr(c["rotated"]), rtol=0, atol=1e-12)


def test_golden_property1_sign_convention(golden):
    """The oracle's 2x2 rotation, read off by rotating unit vectors, reproduces the
    printed products R C = C R of the CommVQ Property 1 proof (this fixes the sign)."""
    c = golden["property1_product"]
    d = 2                                      # one pair, omega_0 = 1: angle = position
    C = np.array([[c["x"], c["y"]], [-c["y"], c["x"]]])
    for ang, want in zip(c["angles"], c["products"]):
        # positions are integers in the cache; use a fractional position to hit
        # the printed angle exactly (the oracle accepts any real position)
        e = np.eye(d)
        cols = O.apply_rope(e, np.array([ang, ang]), theta=10000.0)  # rows = R e_i
        R = cols.T                             # column i is R e_i
        np.testing.assert_allclose(R @ C, _arr(want), atol=1e-12)
        np.testing.assert_allclose(C @ R, _arr(want), atol=1e-12)


def test_golden_gqa_single_token(golden):
    c = golden["gqa_single_token"]
    out = O.decode_attention(_arr(c["q"]), _arr(c["h_k"]), _arr(c["h_v"]), _arr(c["b_k"]),
                             _arr(c["b_v"]), np.array(c["lens"]), rope_theta=c["rope_theta"])
    np.testing.assert_array_equal(out, _arr(c["out"]))


# ------------------------------------------------------------ brute force ---

def _brute(q, h_k, h_v, b_k, b_v, lens, theta):
    """Pure-Python loops with math.fsum; no numpy, no max subtraction."""
    Bsz, Hq, d = len(q), len(q[0]), len(q[0][0])
    G, r, Dg = len(b_k), len(b_k[0]), len(b_k[0][0])
    s = Dg // d
    gqa = Hq // (G * s)
    half = d // 2
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(Bsz)]
    for b in range(Bsz):
        n = lens[b]
        for h in range(Hq):
            j = h // gqa
            g, jl = j // s, j % s
            keys, vals = [], []
            for t in range(n):
                kcol = [math.fsum(h_k[b][g][t][k] * b_k[g][k][jl * d + c] for k in range(r))
                        for c in range(d)]
                vcol = [math.fsum(h_v[b][g][t][k] * b_v[g][k][jl * d + c] for k in range(r))
                        for c in range(d)]
                if theta:
                    rot = list(kcol)
                    for i in range(half):
                        ang = t * theta ** (-2.0 * i / d)
                        x, y = kcol[i], kcol[i + half]
                        rot[i] = x * math.cos(ang) - y * math.sin(ang)
                        rot[i + half] = x * math.sin(ang) + y * math.cos(ang)
                    kcol = rot
                keys.append(kcol)
                vals.append(vcol)
            if n == 0:
                continue
            w = [math.exp(math.fsum(q[b][h][c] * keys[t][c] for c in range(d)) / math.sqrt(d))
                 for t in range(n)]
            tot = math.fsum(w)
            for c in range(d):
                out[b][h][c] = math.fsum(w[t] * vals[t][c] for t in range(n)) / tot
    return out


@pytest.mark.parametrize("theta", [0.0, 10000.0, 500000.0])
@pytest.mark.parametrize("shape", [
    # (B, Hq, Hkv, d, G, r, L)
    (2, 4, 2, 8, 1, 4, 7),      # one group over both KV heads (joint), GQA 2
    (1, 4, 4, 4, 2, 3, 6),      # MHA, two groups of two heads, odd rank
    (2, 6, 2, 6, 2, 5, 5),      # GQA 3, groups of one head
])
def test_brute_force_tiny(shape, theta):
    Bsz, Hq, Hkv, d, G, r, L = shape
    s = Hkv // G
    rng = np.random.default_rng(1234 + sum(shape))
    q = rng.standard_normal((Bsz, Hq, d))
    h_k = rng.standard_normal((Bsz, G, L, r))
    h_v = rng.standard_normal((Bsz, G, L, r))
    b_k = rng.standard_normal((G, r, s * d)) / math.sqrt(r)
    b_v = rng.standard_normal((G, r, s * d)) / math.sqrt(r)
    lens = np.array([L, L - 3][:Bsz])
    want = _brute(q.tolist(), h_k.tolist(), h_v.tolist(), b_k.tolist(), b_v.tolist(),
                  lens.tolist(), theta)
    got = O.decode_attention(q, h_k, h_v, b_k, b_v, lens, rope_theta=theta)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


def test_brute_force_zero_and_one_length():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 2, 4))
    h_k = rng.standard_normal((3, 1, 5, 3))
    h_v = rng.standard_normal((3, 1, 5, 3))
    b_k = rng.standard_normal((1, 3, 8))
    b_v = rng.standard_normal((1, 3, 8))
    lens = np.array([0, 1, 5])
    got = O.decode_attention(q, h_k, h_v, b_k, b_v, lens, rope_theta=10000.0)
    want = _brute(q.tolist(), h_k.tolist(), h_v.tolist(), b_k.tolist(), b_v.tolist(),
                  lens.tolist(), 10000.0)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)
    assert np.all(got[0] == 0.0)


# ------------------------------------------------------- library routines ---

@pytest.mark.parametrize("Hq,Hkv,d,L", [(8, 8, 16, 33), (8, 2, 16, 40), (12, 3, 8, 17)])
def test_identity_factors_reduce_to_sdpa(Hq, Hkv, d, L):
    """r = D_g and B = I: Palu attention is ordinary (GQA) attention with K = H_k and
    V = H_v; torch's fp64 scaled_dot_product_attention is the reference."""
    G = Hkv
    rng = np.random.default_rng(Hq * 100 + L)
    q = rng.standard_normal((2, Hq, d))
    h_k = rng.standard_normal((2, G, L, d))
    h_v = rng.standard_normal((2, G, L, d))
    eye = np.broadcast_to(np.eye(d), (G, d, d)).copy()
    got = O.decode_attention(q, h_k, h_v, eye, eye, np.array([L, L]))
    Q = torch.from_numpy(q)[:, :, None, :]                      # [B, Hq, 1, d]
    K = torch.from_numpy(h_k).repeat_interleave(Hq // Hkv, dim=1)
    V = torch.from_numpy(h_v).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, :, 0, :].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,d,L", [(8, 8, 16, 33), (8, 2, 16, 40), (12, 3, 8, 17)])
def test_full_rank_baseline_is_sdpa(Hq, Hkv, d, L):
    """The uncompressed baseline is ordinary GQA decode attention: torch's fp64
    scaled_dot_product_attention over the first len rows is the reference."""
    rng = np.random.default_rng(Hq * 7 + L)
    q = rng.standard_normal((2, Hq, d))
    k = rng.standard_normal((2, Hkv, L, d))
    v = rng.standard_normal((2, Hkv, L, d))
    lens = np.array([L, L // 2])
    got = O.full_rank_attention(q, k, v, lens)
    for b in range(2):
        n = int(lens[b])
        Q = torch.from_numpy(q[b:b + 1])[:, :, None, :]
        K = torch.from_numpy(k[b:b + 1, :, :n]).repeat_interleave(Hq // Hkv, dim=1)
        V = torch.from_numpy(v[b:b + 1, :, :n]).repeat_interleave(Hq // Hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[0, :, 0, :].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-11, atol=1e-12)


def test_full_rank_baseline_edges():
    """Length 0 gives zeros, length 1 returns that token's value row, and the
    latent path with identity factors (r = d, one group per KV head) agrees."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((3, 2, 6, 8))
    v = rng.standard_normal((3, 2, 6, 8))
    lens = np.array([0, 1, 6])
    got = O.full_rank_attention(q, k, v, lens)
    assert np.all(got[0] == 0.0)
    np.testing.assert_allclose(got[1], v[1, [0, 0, 1, 1], 0, :], rtol=0, atol=1e-15)
    eye = np.broadcast_to(np.eye(8), (2, 8, 8)).copy()
    np.testing.assert_allclose(got, O.decode_attention(q, k, v, eye, eye, lens), rtol=1e-12,
                               atol=1e-13)


def test_reconstructed_keys_have_rank_r():
    """K_g = H B is at most rank r (the cache stores r numbers per token and group)."""
    rng = np.random.default_rng(3)
    for r in (3, 8):
        H = rng.standard_normal((40, r))
        B = rng.standard_normal((r, 32))
        sv = np.linalg.svd(O.reconstruct(H, B), compute_uv=False)
        assert np.all(sv[r:] < 1e-12 * sv[0])
        assert sv[r - 1] > 1e-6 * sv[0]


def test_projection_associativity():
    """(x A) B = x (A B): caching the latent and reconstructing later equals the
    full projection with W = A B (Palu response, answer to Q2)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 64))
    A = rng.standard_normal((64, 16))
    B = rng.standard_normal((16, 48))
    lhs = O.reconstruct(O.latent_project(x, A), B)
    rhs = x @ (A @ B)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-11)


# -------------------------------------------------------------- invariants ---

def _rand_case(rng, Bsz=2, Hq=8, Hkv=4, d=16, G=2, r=6, L=20):
    s = Hkv // G
    return dict(q=rng.standard_normal((Bsz, Hq, d)),
                h_k=rng.standard_normal((Bsz, G, L, r)),
                h_v=rng.standard_normal((Bsz, G, L, r)),
                b_k=rng.standard_normal((G, r, s * d)) / math.sqrt(r),
                b_v=rng.standard_normal((G, r, s * d)) / math.sqrt(r),
                lens=np.array([L, L - 7][:Bsz]))


def _absorbed(case, scale=None):
    """No-RoPE attention with B_k moved onto the query, (q B_j^T) H_k^T, and B_v
    applied after the weighted sum, (p H_v) B_v."""
    q, h_k, h_v, b_k, b_v, lens = (case[k] for k in ("q", "h_k", "h_v", "b_k", "b_v", "lens"))
    Bsz, Hq, d = q.shape
    G, r, Dg = b_k.shape
    s = Dg // d
    gqa = Hq // (G * s)
    scale = 1 / math.sqrt(d) if scale is None else scale
    out = np.zeros_like(q)
    for b in range(Bsz):
        n = lens[b]
        for h in range(Hq):
            j = h // gqa
            g, jl = j // s, j % s
            Bk = b_k[g][:, jl * d:(jl + 1) * d]
            Bv = b_v[g][:, jl * d:(jl + 1) * d]
            qt = Bk @ q[b, h]                      # q B_j^T, length r
            z = h_k[b, g, :n] @ qt * scale
            p = np.exp(z - z.max())
            p /= p.sum()
            out[b, h] = (p @ h_v[b, g, :n]) @ Bv
    return out


def test_absorbed_equals_explicit_without_rope():
    case = _rand_case(np.random.default_rng(11))
    got = O.decode_attention(**case, rope_theta=0.0)
    np.testing.assert_allclose(got, _absorbed(case), rtol=1e-12, atol=1e-12)


def test_value_fold():
    """(p H_v) B_v = p (H_v B_v)."""
    rng = np.random.default_rng(2)
    p = rng.random(30)
    p /= p.sum()
    H = rng.standard_normal((30, 7))
    B = rng.standard_normal((7, 12))
    np.testing.assert_allclose((p @ H) @ B, p @ O.reconstruct(H, B), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("theta", [0.0, 1e4])
def test_value_latents_times_bv_is_the_output(theta):
    """u* B_v[g][:, cols(j)] reproduces the attention output head by head
    (GQA, two groups of two KV heads), with and without RoPE."""
    rng = np.random.default_rng(31)
    B, Hq, d, G, r, L = 2, 8, 8, 2, 5, 9
    Dg = 2 * d
    q = rng.standard_normal((B, Hq, d))
    h_k = rng.standard_normal((B, G, L, r))
    h_v = rng.standard_normal((B, G, L, r))
    b_k = rng.standard_normal((G, r, Dg))
    b_v = rng.standard_normal((G, r, Dg))
    lens = np.array([L, 4])
    u = O.decode_value_latents(q, h_k, h_v, b_k, lens, Dg, rope_theta=theta)
    want = O.decode_attention(q, h_k, h_v, b_k, b_v, lens, rope_theta=theta)
    for h in range(Hq):
        g, jl = (h // 2) // 2, (h // 2) % 2
        got = u[:, h] @ b_v[g][:, jl * d:(jl + 1) * d]
        np.testing.assert_allclose(got, want[:, h], rtol=1e-11, atol=1e-12)


def test_value_latents_closed_forms():
    """One token: u* is that token's value latent row; equal value rows: u* is
    that row whatever the weights; length 0: zeros."""
    rng = np.random.default_rng(32)
    q = rng.standard_normal((3, 2, 4))
    h_k = rng.standard_normal((3, 1, 5, 3))
    h_v = rng.standard_normal((3, 1, 5, 3))
    h_v[2, 0, :] = np.array([0.5, -1.25, 2.0])
    b_k = rng.standard_normal((1, 3, 8))
    u = O.decode_value_latents(q, h_k, h_v, b_k, np.array([1, 0, 5]), 8, rope_theta=100.0)
    np.testing.assert_allclose(u[0], np.tile(h_v[0, 0, 0], (2, 1)), rtol=0, atol=1e-15)
    assert np.all(u[1] == 0.0)
    np.testing.assert_allclose(u[2], np.tile([0.5, -1.25, 2.0], (2, 1)), rtol=0, atol=1e-14)


def test_quantize_round_trip_and_symmetry():
    """Each code is within half a step of h / scale (dequantised error at most
    half a scale), the largest magnitude of a row maps to +-127, codes are odd
    under negation, and a row scaled by 2^k keeps its codes."""
    rng = np.random.default_rng(41)
    h = rng.standard_normal((64, 96)).astype(np.float32)
    h[5] *= 300.0
    h[9, 3] = 40.0                                   # an outlier in one row
    codes, scales = O.quantize_rows_i8(h)
    deq = O.dequantize_rows_i8(codes, scales)
    assert np.all(np.abs(deq - h) <= scales[:, None] * (0.5 + 1e-5))
    rows = np.arange(64)
    top = np.argmax(np.abs(h), axis=1)
    np.testing.assert_array_equal(np.abs(codes[rows, top]), 127)
    c2, s2 = O.quantize_rows_i8(-h)
    np.testing.assert_array_equal(c2, -codes)
    np.testing.assert_array_equal(s2, scales)
    c3, s3 = O.quantize_rows_i8(h * np.float32(8.0))
    np.testing.assert_array_equal(c3, codes)
    np.testing.assert_array_equal(s3, scales * np.float32(8.0))


def test_golden_quantize_rows_i4():
    """Hand-derived int4 codes: amax 3.5 -> scale 0.5, codes h / 0.5 rounded
    to nearest even (1.25 -> 2.5 -> 2, 0.75 -> 1.5 -> 2, -0.25 -> -0.5 -> 0),
    clamped to +-7; a zero row stores scale 0."""
    h = np.array([[3.5, 1.25, 0.75, -0.25, -3.5, 0.0, 1.0, -2.75],
                  [0.0] * 8], dtype=np.float32)
    codes, scales = O.quantize_rows_i4(h)
    np.testing.assert_array_equal(codes[0], [7, 2, 2, 0, -7, 0, 2, -6])
    np.testing.assert_array_equal(codes[1], [0] * 8)
    assert scales[0] == np.float32(0.5) and scales[1] == 0.0


def test_quantize_i4_round_trip_and_symmetry():
    """Codes within half a step (dequantised error at most half a scale), the
    row maximum maps to +-7, odd under negation, invariant under 2^k scaling."""
    rng = np.random.default_rng(47)
    h = rng.standard_normal((64, 64)).astype(np.float32)
    h[3] *= 100.0
    codes, scales = O.quantize_rows_i4(h)
    deq = O.dequantize_rows_i8(codes, scales)
    assert np.all(np.abs(deq - h) <= scales[:, None] * (0.5 + 1e-5))
    top = np.argmax(np.abs(h), axis=1)
    np.testing.assert_array_equal(np.abs(codes[np.arange(64), top]), 7)
    c2, _ = O.quantize_rows_i4(-h)
    np.testing.assert_array_equal(c2, -codes)
    c3, s3 = O.quantize_rows_i4(h * np.float32(4.0))
    np.testing.assert_array_equal(c3, codes)
    np.testing.assert_array_equal(s3, scales * np.float32(4.0))
    assert codes.min() >= -7 and codes.max() <= 7


@pytest.mark.parametrize("r", [1, 2, 4, 64, 256])
def test_hadamard_is_sylvester(r):
    """Entry (i, j) of Sylvester's matrix is (-1)^popcount(i & j) (closed form,
    by induction on the block construction); hence symmetric and H H = r I."""
    H = O.hadamard(r)
    i, j = np.meshgrid(np.arange(r), np.arange(r), indexing="ij")
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    np.testing.assert_array_equal(H, (-1.0) ** pop)
    np.testing.assert_array_equal(H @ H, r * np.eye(r))
    with pytest.raises(ValueError):
        O.hadamard(96)


def test_hadamard_quantisation_of_a_spike():
    """A row with one nonzero latent c at index k rotates to c times row k of
    H (all entries +-c): every code is +-127 with the sign of H[k], the scale
    is |c|/127, and the recovered row is the spike again."""
    r, k, c = 64, 5, np.float32(-3.0)
    h = np.zeros((1, r))
    h[0, k] = c
    codes, scales = O.append_rows_i8_hadamard(h)
    np.testing.assert_array_equal(codes[0], (127 * np.sign(c) * O.hadamard(r)[k]).astype(np.int8))
    assert scales[0] == np.float32(3.0) / np.float32(127.0)
    back = O.dequantize_rows_i8_hadamard(codes, scales)
    np.testing.assert_allclose(back[0], h[0], atol=1e-6)


def test_hadamard_round_trip_bound_and_outliers():
    """Rotated rows come back within half a scale step per element (the
    rotation error e H / r has max norm at most |e|_1 / r <= max |e|); on rows
    with an outlier channel the rotated int8 cache loses less than the plain
    one, which is what the transform is for."""
    rng = np.random.default_rng(43)
    h = rng.standard_normal((200, 128))
    h[:, 7] *= 20.0                                  # one outlier channel
    codes, scales = O.append_rows_i8_hadamard(h)
    back = O.dequantize_rows_i8_hadamard(codes, scales)
    rot32 = (h @ O.hadamard(128)).astype(np.float32).astype(np.float64) @ O.hadamard(128) / 128
    assert np.all(np.abs(back - rot32) <= scales[:, None] * (0.5 + 1e-5))
    pc, ps = O.append_rows_i8(h)
    plain = O.dequantize_rows_i8(pc, ps)
    err_rot = np.linalg.norm(back - h) / np.linalg.norm(h)
    err_plain = np.linalg.norm(plain - h) / np.linalg.norm(h)
    assert err_rot < 0.5 * err_plain


def test_softmax_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((5, 33)) * 10
    p = O.softmax(z)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(O.softmax(z + 123.25), p, atol=1e-12)


def test_single_token_returns_its_value():
    case = _rand_case(np.random.default_rng(8))
    case["lens"] = np.array([1, 1])
    got = O.decode_attention(**case, rope_theta=500000.0)
    Bsz, Hq, d = case["q"].shape
    s = case["b_k"].shape[2] // d
    gqa = Hq // (case["b_k"].shape[0] * s)
    for b in range(Bsz):
        for h in range(Hq):
            j = h // gqa
            g, jl = j // s, j % s
            v0 = case["h_v"][b, g, 0] @ case["b_v"][g][:, jl * d:(jl + 1) * d]
            np.testing.assert_allclose(got[b, h], v0, rtol=1e-13, atol=1e-13)


def test_zero_keys_give_mean_of_values():
    case = _rand_case(np.random.default_rng(9))
    case["h_k"][:] = 0.0
    got = O.decode_attention(**case, rope_theta=10000.0)
    Bsz, Hq, d = case["q"].shape
    s = case["b_k"].shape[2] // d
    gqa = Hq // (case["b_k"].shape[0] * s)
    for b in range(Bsz):
        n = case["lens"][b]
        for h in range(Hq):
            j = h // gqa
            g, jl = j // s, j % s
            V = case["h_v"][b, g, :n] @ case["b_v"][g][:, jl * d:(jl + 1) * d]
            np.testing.assert_allclose(got[b, h], V.mean(0), rtol=1e-12, atol=1e-12)


def test_permutation_invariance_without_rope():
    rng = np.random.default_rng(10)
    case = _rand_case(rng)
    case["lens"] = np.array([20, 20])
    base = O.decode_attention(**case, rope_theta=0.0)
    perm = rng.permutation(20)
    case["h_k"] = case["h_k"][:, :, perm]
    case["h_v"] = case["h_v"][:, :, perm]
    np.testing.assert_allclose(O.decode_attention(**case, rope_theta=0.0), base,
                               rtol=1e-12, atol=1e-12)


def test_rope_position_dependence():
    """With RoPE the context order matters (the no-RoPE invariance above is not a
    property of a path that silently skips the rotation)."""
    rng = np.random.default_rng(12)
    case = _rand_case(rng)
    case["lens"] = np.array([20, 20])
    base = O.decode_attention(**case, rope_theta=10000.0)
    perm = rng.permutation(20)
    case["h_k"] = case["h_k"][:, :, perm]
    case["h_v"] = case["h_v"][:, :, perm]
    assert np.max(np.abs(O.decode_attention(**case, rope_theta=10000.0) - base)) > 1e-3


def test_rope_identity_at_zero_norm_and_relative_position():
    rng = np.random.default_rng(13)
    d, theta = 16, 10000.0
    k = rng.standard_normal((1, d))
    qv = rng.standard_normal((1, d))
    np.testing.assert_allclose(O.apply_rope(k, np.array([0]), theta), k, atol=0)
    for m, n in [(3, 11), (100, 7), (4096, 4000)]:
        Rk = O.apply_rope(k, np.array([n]), theta)
        Rq = O.apply_rope(qv, np.array([m]), theta)
        np.testing.assert_allclose(np.linalg.norm(Rk), np.linalg.norm(k), rtol=1e-13)
        lhs = (Rq @ Rk.T).item()
        rhs = (qv @ O.apply_rope(k, np.array([n - m]), theta).T).item()
        assert abs(lhs - rhs) < 1e-10


def test_rope_frequency_schedule():
    """At position 1 the pair (i, i + d/2) is turned by theta^(-2i/d)."""
    d, theta = 8, 10000.0
    for i in range(d // 2):
        e = np.zeros((1, d))
        e[0, i] = 1.0
        rot = O.apply_rope(e, np.array([1]), theta)[0]
        ang = math.atan2(rot[i + d // 2], rot[i])
        assert abs(ang - theta ** (-2.0 * i / d)) < 1e-14
        others = np.delete(rot, [i, i + d // 2])
        assert np.all(others == 0)


# ------------------------------------------------------------ split merge ---

def test_split_merge_algebra():
    """Partial softmax states (m, l, u) of any partition of the context merge to the
    unsplit result: the algebra a split-context kernel relies on."""
    rng = np.random.default_rng(14)
    z = rng.standard_normal(97) * 3
    H = rng.standard_normal((97, 5))
    p = O.softmax(z)
    want = p @ H
    for cuts in ([0, 97], [0, 10, 97], [0, 1, 2, 50, 96, 97], list(range(0, 98, 13)) + [97]):
        ms, ls, us = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b <= a:
                continue
            m = z[a:b].max()
            e = np.exp(z[a:b] - m)
            ms.append(m), ls.append(e.sum()), us.append(e @ H[a:b])
        M = max(ms)
        w = np.exp(np.array(ms) - M)
        got = (w[:, None] * np.array(us)).sum(0) / (w * np.array(ls)).sum()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- append ---

def test_append_rounding_is_fp32_then_bf16_nearest_even():
    """append_rows_bf16 rounds through fp32 to bf16, ties to even: checked on
    hand-picked fp32 bit patterns."""
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exact
        0x3F808000: 0x3F80,   # tie, even stays
        0x3F818000: 0x3F82,   # tie, odd rounds up
        0x3F808001: 0x3F81,   # above tie
        0x3F807FFF: 0x3F80,   # below tie
        0xBF818000: 0xBF82,   # negative tie, odd -> away from zero
    }
    for fbits, want in cases.items():
        v = np.array([fbits], dtype=np.uint32).view(np.float32).astype(np.float64)
        assert int(O.append_rows_bf16(v)[0]) == want, hex(fbits)


def test_append_matches_projection():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    A = rng.standard_normal((32, 12)).astype(np.float32)
    h = O.latent_project(x, A)
    np.testing.assert_allclose(h, x.astype(np.float64) @ A.astype(np.float64), rtol=1e-13)
    bits = O.append_rows_bf16(h)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - h) <= np.abs(h) * 2.0 ** -8)


# -------------------------------------------------- bf16 storage widening ---

def test_to_f64_bf16_bit_patterns():
    """A bf16 value is the fp32 number whose upper 16 bits are its bits.
    Hand-derived: 0x3F80 is sign 0, exponent 127, mantissa 0 -> 1.0; 0xBF82 is
    -(1 + 2/128) = -1.015625; 0x0001 is the smallest subnormal, 2^-126 * 2^-7
    = 2^-133; 0x7F80 is +inf; 0x4049 is 2 * (1 + 73/128) = 3.140625; 0x8000 is
    -0.0. Also a cross-check against torch's own bfloat16 -> float64 widening."""
    bits = np.array([0x3F80, 0xBF82, 0x0001, 0x7F80, 0x4049, 0x8000], dtype=np.uint16)
    want = [1.0, -1.015625, 2.0 ** -133, math.inf, 3.140625, -0.0]
    got = O.to_f64(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and math.copysign(1.0, g) == math.copysign(1.0, w), (g, w)
    rng = np.random.default_rng(50)
    many = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    many = many[(many & 0x7F80) != 0x7F80]            # finite patterns only
    ref = torch.from_numpy(many.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.to_f64(many), ref)


def _bf16_bits(values):
    """bf16 bits of values that are exactly representable in bf16: the upper
    half of their fp32 encoding (struct packing, independent of the oracle)."""
    import struct
    out = []
    for v in np.asarray(values, dtype=np.float64).ravel():
        w = struct.unpack("<I", struct.pack("<f", float(v)))[0]
        assert w & 0xFFFF == 0, v
        out.append(w >> 16)
    return np.array(out, dtype=np.uint16).reshape(np.shape(values))


def test_brute_force_on_bf16_storage():
    """The oracle fed bf16 bit patterns (every input of the bf16 workloads
    reaches it so) gives the brute-force result of the values those bits
    hold: inputs are multiples of 1/16 in [-4, 4), exact in bf16."""
    Bsz, Hq, Hkv, d, G, r, L = 2, 4, 2, 8, 1, 4, 6
    rng = np.random.default_rng(51)
    draw = lambda *shape: rng.integers(-64, 64, size=shape) / 16.0
    q, h_k, h_v = draw(Bsz, Hq, d), draw(Bsz, G, L, r), draw(Bsz, G, L, r)
    b_k, b_v = draw(G, r, Hkv // G * d) / 4, draw(G, r, Hkv // G * d) / 4
    lens = np.array([L, 3])
    want = _brute(q.tolist(), h_k.tolist(), h_v.tolist(), b_k.tolist(), b_v.tolist(),
                  lens.tolist(), 10000.0)
    got = O.decode_attention(_bf16_bits(q), _bf16_bits(h_k), _bf16_bits(h_v), _bf16_bits(b_k),
                             _bf16_bits(b_v), lens, rope_theta=10000.0)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


# ------------------------------------------- quantised cache writes (rows) ---
#
# Per-token quantisation of the latents (Palu author response to reviewer
# Fsn9, W1/W2; "Avg. Bits" with a scale shared by a group, answer to Q4). The
# kernel's row is an fp32 sum, so the oracle rounds the exact row to fp32 once
# and takes every decision on that fp32 row. The rows below hold elements whose
# exact value and fp32 rounding fall on different sides of a rounding decision.

def test_append_rows_i8_hand_row():
    """Exact row [127 + 2^-40, 2.5 + 2^-30, 2.5078125, -63.5, 0.5 - 2^-40, -1.5,
    0, 126.5] rounds to the fp32 row [127, 2.5, 2.5078125, -63.5, 0.5, -1.5, 0,
    126.5] (the added terms are far below half an fp32 ulp). amax = 127, so
    scale = 127/127 = 1 and the multiplier 127/127 = 1; codes are the
    nearest-even integers of the fp32 row: [127, 2, 3, -64, 0, -2, 0, 126]. The
    exact value 2.5 + 2^-30 would give 3, and 2.5078125 rounded to bf16 first
    (a tie, to the even 2.5) would give 2."""
    h = np.array([[127 + 2.0 ** -40, 2.5 + 2.0 ** -30, 2.5078125, -63.5, 0.5 - 2.0 ** -40,
                   -1.5, 0.0, 126.5]])
    codes, scales = O.append_rows_i8(h)
    assert codes.dtype == np.int8
    np.testing.assert_array_equal(codes[0], [127, 2, 3, -64, 0, -2, 0, 126])
    assert scales.dtype == np.float32 and scales[0] == np.float32(1.0)
    # the same row ten times larger: amax 1270 (exact in fp32), scale 10,
    # multiplier fl(127/1270) = fl(0.1); every code is then one fp32 product
    # away from the integer or tie it was before, computed here by hand
    h10 = np.array([[1270.0, 25.0, 5.0, -635.0, 0.0, 12.5, -12.5, 1265.0]])
    codes, scales = O.append_rows_i8(h10)
    inv = np.float32(127.0) / np.float32(1270.0)                  # fl(0.1)
    prods = [np.float32(v) * inv for v in h10[0]]
    np.testing.assert_array_equal(codes[0], [int(np.rint(p)) for p in prods])
    assert scales[0] == np.float32(1270.0) / np.float32(127.0)
    assert list(codes[0][:4]) == [127, 2, 0, -64]


def test_append_rows_i4_hand_row():
    """int4: exact row [7 + 2^-40, 2.5 + 2^-30, -3.5, 1.5, 0.5 - 2^-40, 6.5, -7,
    0.25] -> fp32 [7, 2.5, -3.5, 1.5, 0.5, 6.5, -7, 0.25]; amax 7, scale 7/7 =
    1, multiplier 1; codes nearest-even: [7, 2, -4, 2, 0, 6, -7, 0] (15
    levels). An int8 quantiser would give 127 for the first element."""
    h = np.array([[7 + 2.0 ** -40, 2.5 + 2.0 ** -30, -3.5, 1.5, 0.5 - 2.0 ** -40, 6.5, -7.0,
                   0.25]])
    codes, scales = O.append_rows_i4(h)
    np.testing.assert_array_equal(codes[0], [7, 2, -4, 2, 0, 6, -7, 0])
    assert scales[0] == np.float32(1.0)
    z_codes, z_scales = O.append_rows_i4(np.zeros((1, 8)))
    assert np.all(z_codes == 0) and z_scales[0] == 0.0


def test_hadamard_i4_quantisation_of_a_spike():
    """Rotated int4 write of a row with one nonzero latent c at index k: h H_r
    is c times row k of Sylvester's matrix (entries +-c), so every code is
    +-7 with the sign of c H[k], the scale is |c|/7, and rotating the
    dequantised row back gives the spike."""
    r, k, c = 64, 9, np.float32(-3.0)
    h = np.zeros((1, r))
    h[0, k] = c
    codes, scales = O.append_rows_i4_hadamard(h)
    i, j = k, np.arange(r)
    sign_row = (-1.0) ** np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    np.testing.assert_array_equal(codes[0], (7 * np.sign(c) * sign_row).astype(np.int8))
    assert scales[0] == np.float32(3.0) / np.float32(7.0)
    back = O.dequantize_rows_i8_hadamard(codes, scales)
    np.testing.assert_allclose(back[0], h[0], atol=1e-6)
