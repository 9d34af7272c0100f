"""CPU oracle for decode attention over a low-rank (Palu-style) latent KV cache.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

What it computes, in fp64, the plain way (no tiling, no fusion, no reordering
beyond what the definitions state):

  * Cache write, Palu author response on OpenReview, answer to Q2 (ESPACE):
    inference runs a down-projection h = x A and a reconstruction y = h B.
  * Key reconstruction, same page, "Why Palu Requires Fewer Global Memory
    Access": the cached latent H_i (L x r) and the matrix B_i (r x d_h) give
    the full key K_i = H_i B_i; the baseline score is the GEMV q_i K_i^T.
  * Grouped-head decomposition (G-LRD), same page, "Quantitive Analysis" and
    the Qwen2.5 follow-up: heads are decomposed per group; one group spanning
    all heads is the joint decomposition (J-LRD).
  * Value path, same page, clarification of W1: the value matrix is never
    rebuilt; its reconstruction matrix is applied after the attention-weighted
    sum. The oracle nevertheless rebuilds V = H_v B_v explicitly and forms
    p V, which is the same quantity by associativity.
  * Attention, CurDKV author response (page "klmc4fwPLd"), motivation of
    value-guided compression: out = softmax(Q K^T / C) V with C a constant
    set by the dimension; here C = sqrt(head_dim).
  * Rotary embedding, CommVQ author response (page "sbbyCB39HN"), proof of
    Property 1: the rotation of a 2-D pair at position m and frequency
    theta_i is [[cos m theta_i, -sin m theta_i], [sin m theta_i, cos m theta_i]].

Readings where the pages are silent (each listed in the design notes):
  * frequencies omega_i = theta ** (-2 i / d), i in [0, d/2), and the pair
    rotated together is (i, i + d/2) of a head's d channels. No page fixes
    the pairing (the interleaved pairs (2i, 2i+1) fit them equally well), so
    apply_rope is parity unpinned as to the pairing: its pins fix the sign,
    the frequency schedule and the rotation's properties, and both sides
    share the pairing;
  * RoPE acts on reconstructed keys at positions 0..len-1; q arrives already
    position-encoded;
  * group g holds KV heads g*s .. g*s+s-1; KV head g*s+jl uses columns
    jl*d .. (jl+1)*d of B_g; query head h reads KV head h // (Hq / Hkv);
  * a sequence of length 0 yields a zero output.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = ["to_f64", "latent_project", "append_rows_bf16", "quantize_rows_i8",
           "dequantize_rows_i8", "append_rows_i8", "quantize_rows_i4", "append_rows_i4",
           "hadamard", "append_rows_i8_hadamard", "append_rows_i4_hadamard",
           "dequantize_rows_i8_hadamard", "reconstruct", "rope_angles", "apply_rope", "softmax",
           "attend", "decode_attention", "full_rank_attention", "decode_value_latents",
           "head_layout"]


# ---------------------------------------------------------------- inputs ---

def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of a stored tensor: fp32 values, or bf16 given as uint16 bits
    (a bf16 value is the fp32 whose upper 16 bits are those bits)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------ cache write ---

def latent_project(x: np.ndarray, a: np.ndarray) -> np.ndarray:
    """h = x A (ESPACE answer, Q2): x [B, d_model], A [d_model, G*r] -> [B, G*r]."""
    return to_f64(x) @ to_f64(a)


def append_rows_bf16(h64: np.ndarray) -> np.ndarray:
    """Store fp64 latents the way a bf16 cache holds them when the sum is formed in
    fp32: round to the nearest fp32, then to the nearest bf16 (ties to even).
    Returns uint16 bits."""
    f = np.asarray(h64, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rest = u & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def quantize_rows_i8(h32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token int8 quantisation of latent rows (the pages list per-token
    quantisation of the low-rank latents as the follow-on lever; reading taken
    here: symmetric, one scale per cached row of r latents).

    With fp32 arithmetic throughout (the kernel's precision, so that both sides
    take the same integer decisions): amax = max |h|, scale = amax / 127,
    inv = 127 / amax (each a correctly rounded fp32 division), code =
    round-to-nearest-even(h * inv) clamped to [-127, 127]. A row of zeros gets
    scale 0 and codes 0. Returns (int8 codes [..., r], fp32 scales [...]).
    """
    h = np.asarray(h32, dtype=np.float32)
    amax = np.max(np.abs(h), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
    scale = np.where(nz, safe / np.float32(127.0), np.float32(0.0)).astype(np.float32)
    inv = np.where(nz, np.float32(127.0) / safe, np.float32(0.0)).astype(np.float32)
    prod = (h * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return codes, scale


def dequantize_rows_i8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """h = code * scale, exactly, in fp64."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def append_rows_i8(h64: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantised cache write: the latent row as the kernel forms it (the fp32
    sum, here the exact value rounded once to fp32), then quantize_rows_i8."""
    return quantize_rows_i8(np.asarray(h64, dtype=np.float64).astype(np.float32))


def quantize_rows_i4(h32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token int4 quantisation of latent rows (the other width the
    follow-on lever names; reading taken here: symmetric, 15 levels): in fp32,
    amax = max |h|, scale = amax / 7, inv = 7 / amax (correctly rounded),
    code = round-to-nearest-even(h * inv) clamped to [-7, 7]; a row of zeros
    gets scale 0 and codes 0. Returns (int8 codes in [-7, 7], fp32 scales)."""
    h = np.asarray(h32, dtype=np.float32)
    amax = np.max(np.abs(h), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
    scale = np.where(nz, safe / np.float32(7.0), np.float32(0.0)).astype(np.float32)
    inv = np.where(nz, np.float32(7.0) / safe, np.float32(0.0)).astype(np.float32)
    prod = (h * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -7, 7).astype(np.int8)
    return codes, scale


def append_rows_i4(h64: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """int4 cache write: the exact row rounded once to fp32, then quantize_rows_i4."""
    return quantize_rows_i4(np.asarray(h64, dtype=np.float64).astype(np.float32))


# -------------------------------------------- Hadamard-rotated int8 cache ---
#
# The Palu author responses name fusing a Hadamard transform as one of the
# quantisation-friendly enhancements of the latent cache (answer to Q2,
# ESPACE; the reply on LASER lists the same enhancements), next to per-token
# quantisation of the latents (reply to reviewer Fsn9 on W1/W2). Reading
# taken here (the pages give neither the matrix nor where it is applied): each latent row h (length r, a power
# of two) is rotated by the Sylvester Hadamard matrix H_r before per-token
# quantisation, h'' = h H_r, so that an outlier channel is spread over all r
# codes; since H_r H_r = r I, the row is recovered as h = h'' H_r / r. The
# rotation is orthogonal up to the factor r, so attention over the recovered
# rows is attention over the original ones, up to quantisation.

def hadamard(r: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order r (a power of two), entries +-1:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if r < 1 or r & (r - 1):
        raise ValueError("r must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < r:
        h = np.block([[h, h], [h, -h]])
    return h


def append_rows_i8_hadamard(h64: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantised cache write of rotated rows: h'' = h H_r formed exactly and
    rounded once to fp32 (the kernel's precision for the integer decisions),
    then quantize_rows_i8. Returns (codes of h'', scales of h'')."""
    h = np.asarray(h64, dtype=np.float64)
    rot = h @ hadamard(h.shape[-1])
    return quantize_rows_i8(rot.astype(np.float32))


def dequantize_rows_i8_hadamard(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Latent rows of a rotated int8 (or int4) cache: (code * scale) H_r / r, in fp64."""
    r = codes.shape[-1]
    return dequantize_rows_i8(codes, scales) @ hadamard(r) / r


def append_rows_i4_hadamard(h64: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Rotated int4 cache write: h H_r formed exactly, rounded once to fp32,
    then quantize_rows_i4."""
    h = np.asarray(h64, dtype=np.float64)
    return quantize_rows_i4((h @ hadamard(h.shape[-1])).astype(np.float32))


# --------------------------------------------------------- reconstruction ---

def reconstruct(h: np.ndarray, b: np.ndarray) -> np.ndarray:
    """K = H B ("Why Palu Requires Fewer Global Memory Access"): H [n, r], B [r, D_g]."""
    return to_f64(h) @ to_f64(b)


# ------------------------------------------------------------------ RoPE ---

def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """phi[t, i] = positions[t] * theta ** (-2 i / d), i in [0, d/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]


def apply_rope(k: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate each pair (k[:, i], k[:, i + d/2]) of the rows of k [n, d] by the
    2x2 rotation [[cos phi, -sin phi], [sin phi, cos phi]] (CommVQ response,
    Property 1 proof). theta == 0 means no rotation."""
    k = np.asarray(k, dtype=np.float64)
    if theta == 0:
        return k.copy()
    half = k.shape[1] // 2
    phi = rope_angles(positions, k.shape[1], theta)
    c, s = np.cos(phi), np.sin(phi)
    x, y = k[:, :half], k[:, half:]
    return np.concatenate([c * x - s * y, s * x + c * y], axis=1)


# ------------------------------------------------------------- attention ---

def softmax(z: np.ndarray) -> np.ndarray:
    """Textbook softmax over the last axis (max subtracted for range only)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for one query row q [d], K [n, d], V [n, d]."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    return softmax((K @ q) * scale) @ V


def head_layout(n_q_heads: int, n_groups: int, rank: int, group_dim: int,
                head_dim: int) -> Tuple[int, int, int]:
    """(s, gqa, n_kv_heads) from the tensor shapes; raises on inconsistent shapes."""
    if group_dim % head_dim:
        raise ValueError("group_dim must be a multiple of head_dim")
    s = group_dim // head_dim
    n_kv = n_groups * s
    if n_q_heads % n_kv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return s, n_q_heads // n_kv, n_kv


def decode_attention(q: np.ndarray, h_k: np.ndarray, h_v: np.ndarray, b_k: np.ndarray,
                     b_v: np.ndarray, lens: np.ndarray, *, rope_theta: float = 0.0,
                     scale: Optional[float] = None,
                     select: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """Single-token decode attention over the latent cache, with K and V rebuilt
    explicitly.

    q [B, Hq, d]; h_k, h_v [B, G, L_cap, r]; b_k, b_v [G, r, D_g]; lens [B].
    Returns fp64 out [B, Hq, d]. With select = [(b, h), ...] only those rows are
    computed and the rest are NaN (sampled checks at full size).
    """
    Bsz, Hq, d = q.shape
    G, r, Dg = b_k.shape
    s, gqa, _ = head_layout(Hq, G, r, Dg, d)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.full((Bsz, Hq, d), np.nan)
    if select is None:
        wanted = {(b, h) for b in range(Bsz) for h in range(Hq)}
    else:
        wanted = {(int(b), int(h)) for b, h in select}
    bk_all, bv_all = to_f64(b_k), to_f64(b_v)
    for b in range(Bsz):
        n = int(lens[b])
        for g in range(G):
            heads = [h for h in range(Hq) if (b, h) in wanted and (h // gqa) // s == g]
            if not heads:
                continue
            if n == 0:
                for h in heads:
                    out[b, h] = 0.0
                continue
            Kg = reconstruct(h_k[b, g, :n], bk_all[g])        # [n, D_g]
            Vg = reconstruct(h_v[b, g, :n], bv_all[g])        # [n, D_g]
            pos = np.arange(n)
            for h in heads:
                j = h // gqa
                jl = j - g * s
                Kj = apply_rope(Kg[:, jl * d:(jl + 1) * d], pos, rope_theta)
                Vj = Vg[:, jl * d:(jl + 1) * d]
                out[b, h] = attend(to_f64(q[b, h]), Kj, Vj, scale)
    return out


def full_rank_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lens: np.ndarray, *,
                        scale: Optional[float] = None,
                        select: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """The uncompressed baseline the pages measure against ("Why Palu Requires
    Fewer Global Memory Access": the baseline reads the full key K_i and forms
    q_i K_i^T): ordinary decode attention over full keys and values.

    q [B, Hq, d]; k, v [B, Hkv, L_cap, d] (keys already position-encoded);
    lens [B]. Query head h reads KV head h // (Hq / Hkv). Returns fp64
    [B, Hq, d]; with select only those (b, h) rows are computed (rest NaN).
    """
    Bsz, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    gqa = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.full((Bsz, Hq, d), np.nan)
    wanted = None if select is None else {(int(b), int(h)) for b, h in select}
    for b in range(Bsz):
        n = int(lens[b])
        for h in range(Hq):
            if wanted is not None and (b, h) not in wanted:
                continue
            j = h // gqa
            out[b, h] = attend(to_f64(q[b, h]), to_f64(k[b, j, :n]), to_f64(v[b, j, :n]), scale)
    return out


def decode_value_latents(q: np.ndarray, h_k: np.ndarray, h_v: np.ndarray, b_k: np.ndarray,
                         lens: np.ndarray, group_dim: int, *, rope_theta: float = 0.0,
                         scale: Optional[float] = None) -> np.ndarray:
    """The attention-weighted sum of value latents, u*[b, h] = sum_t p_t h_v[b, g, t]
    (Palu author response, clarification of W1: the value reconstruction matrix
    acts after this sum, so it can be fused with the output projection: the
    result times B_v[g][:, cols(j)] is the attention output of decode_attention).

    q [B, Hq, d]; h_k, h_v [B, G, L_cap, r]; b_k [G, r, D_g]; group_dim = D_g.
    The weights p_t come from the same rebuilt (and rotated) keys as in
    decode_attention. Returns fp64 [B, Hq, r]; length 0 gives zeros.
    """
    Bsz, Hq, d = q.shape
    G, r, Dg = b_k.shape
    if Dg != group_dim:
        raise ValueError("b_k does not match group_dim")
    s, gqa, _ = head_layout(Hq, G, r, Dg, d)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.zeros((Bsz, Hq, r))
    bk_all = to_f64(b_k)
    for b in range(Bsz):
        n = int(lens[b])
        if n == 0:
            continue
        for g in range(G):
            Kg = reconstruct(h_k[b, g, :n], bk_all[g])        # [n, D_g]
            Hv = to_f64(h_v[b, g, :n])                        # [n, r]
            pos = np.arange(n)
            for h in range(g * s * gqa, (g + 1) * s * gqa):
                jl = h // gqa - g * s
                Kj = apply_rope(Kg[:, jl * d:(jl + 1) * d], pos, rope_theta)
                p_t = softmax((Kj @ to_f64(q[b, h])) * scale)
                out[b, h] = p_t @ Hv
    return out
