"""Seeded synthetic inputs for low-rank latent-KV decode attention.

This module is the only code shared by the CPU oracle and the HIP path. It
draws random numbers and stores them in the two storage formats the path
accepts (fp32, or bf16 held as raw uint16 bits); it contains none of the
method's arithmetic (no projection, reconstruction, rotation or softmax).

Shapes follow the notation of the Palu author response on OpenReview
("Why Palu Requires Fewer Global Memory Access"): per token and per head
group a latent h in R^r is cached, and a group's reconstruction matrix B is
r x D_g (D_g = heads_per_group * head_dim).

Layouts (row-major, last index fastest):
    q        [B, Hq, d]
    h_k, h_v [B, G, L_cap, r]
    b_k, b_v [G, r, D_g]
    lens     [B] int32
    x        [B, d_model]          (d_model = Hq * d)
    a_k, a_v [d_model, G * r]
    pos      [B] int32             (row written by the latent append)

Distributions: latents, q and x are N(0, 1); B is N(0, 1/r) (the second
argument is a variance, so a reconstructed key has unit variance); A is
N(0, 1/d_model). Draws are made in fp32 and, for bf16 workloads, rounded to
the nearest bf16 (ties to even) once, here, so that both sides see the same
bits. Each tensor has its own child stream of numpy's PCG64 seeded from
(seed, tensor index), so a tensor can be drawn without drawing the others.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = ["Config", "CONFIGS", "generate", "f32_to_bf16_bits", "bf16_bits_to_f32",
           "poison_tail", "latent_bytes"]

# child-stream index of every tensor: fixed, so adding a tensor never changes
# the bits of another
_STREAM = {"q": 0, "h_k": 1, "h_v": 2, "b_k": 3, "b_v": 4, "lens": 5,
           "outlier": 6, "x": 7, "a_k": 8, "a_v": 9, "pos": 10, "k_full": 11, "v_full": 12,
           "k_i8": 13, "v_i8": 14, "sk": 15, "sv": 16, "k_i4": 17, "v_i4": 18, "sk_i4": 19,
           "sv_i4": 20}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_groups: int
    rank: int
    max_ctx: int                 # L_cap: rows reserved per (b, g)
    dtype: str                   # "f32" or "bf16"
    rope_theta: float            # 0 means no rotary embedding
    modes: Tuple[str, ...]       # "reconstruct" and/or "absorbed"
    ragged: Optional[Tuple[int, int]] = None   # inclusive bounds of len[b]
    outlier_frac: float = 0.0    # fraction of latent channels scaled
    outlier_scale: float = 1.0
    seed: int = 0

    # ---- derived sizes -------------------------------------------------
    @property
    def heads_per_group(self) -> int:          # s
        return self.n_kv_heads // self.n_groups

    @property
    def group_dim(self) -> int:                # D_g
        return self.heads_per_group * self.head_dim

    @property
    def q_per_group(self) -> int:              # n_q
        return self.n_q_heads // self.n_groups

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def d_model(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def compression(self) -> float:
        """Fraction of the per-head-group KV size removed: 1 - r / D_g."""
        return 1.0 - self.rank / self.group_dim

    def scaled(self, **kw) -> "Config":
        """Same head structure with some sizes replaced (parity-test variants)."""
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[int, Config] = {
    1: Config("tiny", batch=1, n_q_heads=8, n_kv_heads=8, head_dim=64, n_groups=4,
              rank=32, max_ctx=512, dtype="f32", rope_theta=0.0,
              modes=("reconstruct", "absorbed"), seed=1),
    2: Config("llama2_7b_mha", batch=16, n_q_heads=32, n_kv_heads=32, head_dim=128,
              n_groups=8, rank=256, max_ctx=4096, dtype="bf16", rope_theta=1e4,
              modes=("reconstruct",), seed=2),
    3: Config("llama3_8b_gqa", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128,
              n_groups=2, rank=256, max_ctx=32768, dtype="bf16", rope_theta=5e5,
              modes=("reconstruct", "absorbed"), seed=3),
    4: Config("long_ctx_outliers", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
              n_groups=2, rank=128, max_ctx=131072, dtype="bf16", rope_theta=5e5,
              modes=("reconstruct",), outlier_frac=0.01, outlier_scale=20.0, seed=4),
    5: Config("ragged_jlrd", batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
              n_groups=1, rank=512, max_ctx=16384, dtype="bf16", rope_theta=5e5,
              modes=("reconstruct",), ragged=(1024, 16384), seed=5),
}


def latent_bytes(cfg: Config, lens: np.ndarray) -> int:
    """Bytes of h_k plus h_v that one decode step must read (valid rows only)."""
    elem = 4 if cfg.dtype == "f32" else 2
    return int(2 * int(np.sum(lens, dtype=np.int64)) * cfg.n_groups * cfg.rank * elem)


# ---- storage-format helpers (bit packing, not arithmetic of the method) ---

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16, ties to even; returns uint16 bits.
    Inputs here are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _STREAM[name]]))


def _normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    a = _rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def generate(cfg: Config, *, seed: Optional[int] = None, parts=("decode",),
             lens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Draw one workload.

    parts: "decode" -> q, h_k, h_v, b_k, b_v, lens; "append" -> x, a_k, a_v, pos;
    "full" -> k_full, v_full [B, Hkv, L_cap, d] (the uncompressed baseline's
    cache, same q and lens as "decode", which it needs); "i8" -> k_i8, v_i8
    int8 [B, G, L_cap, r] (codes uniform in [-127, 127]) and sk, sv fp32
    [B, G, L_cap] (scales uniform in [0.005, 0.025)): an int8 latent cache;
    "i4" -> k_i4, v_i4 int8 [B, G, L_cap, r] (codes uniform in [-7, 7]) and
    sk_i4, sv_i4 (scales uniform in [0.1, 0.45)): an int4 latent cache, codes
    in row order (both caches span latents up to about 3.2 in magnitude).
    lens overrides the drawn lengths (edge-case tests). Values are fp32 arrays or
    uint16 bf16 bits, per cfg.dtype; lens and pos are int32.
    """
    seed = cfg.seed if seed is None else seed
    B, Hq, d, G, r, L = (cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.n_groups,
                         cfg.rank, cfg.max_ctx)
    out: Dict[str, np.ndarray] = {}
    if "decode" in parts:
        out["q"] = _store(_normal(seed, "q", (B, Hq, d)), cfg.dtype)
        # outlier channels: round(frac * G * r) of the G*r latent channels,
        # chosen separately for h_k and h_v, scaled in fp32 before rounding
        n_out = int(round(cfg.outlier_frac * G * r))
        orng = _rng(seed, "outlier")
        for name in ("h_k", "h_v"):
            h = _normal(seed, name, (B, G, L, r))
            if n_out:
                ch = orng.choice(G * r, size=n_out, replace=False)
                for c in ch:
                    h[:, c // r, :, c % r] *= np.float32(cfg.outlier_scale)
            out[name] = _store(h, cfg.dtype)
            del h
        for name in ("b_k", "b_v"):
            out[name] = _store(_normal(seed, name, (G, r, cfg.group_dim), 1.0 / math.sqrt(r)),
                               cfg.dtype)
        if lens is None:
            if cfg.ragged is not None:
                lo, hi = cfg.ragged
                lens = _rng(seed, "lens").integers(lo, hi + 1, size=B)
            else:
                lens = np.full(B, L)
        lens = np.asarray(lens, dtype=np.int32)
        if lens.shape != (B,) or lens.min(initial=0) < 0 or lens.max(initial=0) > L:
            raise ValueError("lens must be [B] with 0 <= len <= max_ctx")
        out["lens"] = lens
    if "full" in parts:
        Hkv = cfg.n_kv_heads
        for name in ("k_full", "v_full"):
            out[name] = _store(_normal(seed, name, (B, Hkv, L, d)), cfg.dtype)
    if "i8" in parts:
        for name in ("k_i8", "v_i8"):
            out[name] = _rng(seed, name).integers(-127, 128, size=(B, G, L, r)).astype(np.int8)
        for name in ("sk", "sv"):
            u = _rng(seed, name).random(size=(B, G, L), dtype=np.float32)
            out[name] = (np.float32(0.005) + np.float32(0.02) * u).astype(np.float32)
    if "i4" in parts:
        for name in ("k_i4", "v_i4"):
            out[name] = _rng(seed, name).integers(-7, 8, size=(B, G, L, r)).astype(np.int8)
        for name in ("sk_i4", "sv_i4"):
            u = _rng(seed, name).random(size=(B, G, L), dtype=np.float32)
            out[name] = (np.float32(0.1) + np.float32(0.35) * u).astype(np.float32)
    if "append" in parts:
        dm = cfg.d_model
        out["x"] = _store(_normal(seed, "x", (B, dm)), cfg.dtype)
        out["a_k"] = _store(_normal(seed, "a_k", (dm, G * r), 1.0 / math.sqrt(dm)), cfg.dtype)
        out["a_v"] = _store(_normal(seed, "a_v", (dm, G * r), 1.0 / math.sqrt(dm)), cfg.dtype)
        out["pos"] = _rng(seed, "pos").integers(0, L, size=B).astype(np.int32)
    return out


def poison_tail(h: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """Copy of a latent cache [B, G, L, r] whose rows at or beyond len[b] are NaN,
    so that any read past the valid context shows up in the output."""
    h = h.copy()
    nan = np.uint16(0x7FC0) if h.dtype == np.uint16 else np.float32("nan")
    for b, n in enumerate(lens):
        h[b, :, int(n):, :] = nan
    return h
