"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
calling the library through its binding, and the error metrics."""
from __future__ import annotations

import numpy as np
import torch

import rank_compressed_kv_amd as P

MAX_ABS = 2e-2      # per-element bound for the bf16 workloads
REL_L2 = 5e-3       # ||gpu - oracle||_2 / ||oracle||_2


def dev(a: np.ndarray) -> torch.Tensor:
    """Seeded host array -> device tensor with the same bits (uint16 = bf16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype in (np.int32, np.int8, np.uint8):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_decode(cfg, t, mode, *, rope_theta=None, split_tokens=0, lens=True, h_k=None, h_v=None):
    theta = (cfg.rope_theta if mode == "reconstruct" else 0.0) if rope_theta is None else rope_theta
    q, bk, bv = dev(t["q"]), dev(t["b_k"]), dev(t["b_v"])
    hk = dev(t["h_k"] if h_k is None else h_k)
    hv = dev(t["h_v"] if h_v is None else h_v)
    ln = dev(t["lens"]) if lens else None
    out = P.decode_attention(q, hk, hv, bk, bv, ln, n_kv_heads=cfg.n_kv_heads, mode=mode,
                             rope_theta=theta, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), theta


def errors(got: np.ndarray, want: np.ndarray):
    mask = ~np.isnan(want)
    g, w = got[mask], want[mask]
    diff = np.abs(g - w)
    max_abs = float(diff.max()) if diff.size else 0.0
    den = float(np.linalg.norm(w))
    rel = float(np.linalg.norm(g - w) / den) if den > 0 else float(np.linalg.norm(g - w))
    return max_abs, rel


def assert_close(got, want, *, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    assert np.all(np.isfinite(got[~np.isnan(want)])), f"{what}: non-finite output"
    ma, rel = errors(got, want)
    assert ma <= max_abs and rel <= rel_l2, f"{what}: max|d|={ma:.3e} relL2={rel:.3e}"
    return ma, rel


def code_bounds(e, E, amax_lo, amax_hi, qmax):
    """Range of codes rint(S * fl(qmax / A)) over every fp32 sum S within E of
    the exact value e and every row maximum A in [amax_lo, amax_hi] (rounding
    is monotone, so the corners bound it); returns (lo, hi) codes."""
    eps = 2.0 ** -23
    inv_lo = qmax / amax_hi * (1 - eps)
    inv_hi = qmax / amax_lo * (1 + eps) if amax_lo > 0 else np.inf
    corners = np.stack([(e - E) * inv_lo, (e - E) * inv_hi, (e + E) * inv_lo, (e + E) * inv_hi])
    with np.errstate(invalid="ignore"):
        lo = np.nanmin(corners, 0) * (1 - np.sign(np.nanmin(corners, 0)) * eps)
        hi = np.nanmax(corners, 0) * (1 + np.sign(np.nanmax(corners, 0)) * eps)
    return np.clip(np.rint(lo), -qmax, qmax), np.clip(np.rint(hi), -qmax, qmax)
