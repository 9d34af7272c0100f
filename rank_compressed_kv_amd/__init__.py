"""Python binding of libpalu: decode attention over a low-rank latent KV cache
on MI355X (gfx950).

This module only marshals arguments: it checks tensor shapes, dtypes and
devices against the descriptor, then calls the C ABI of include/palu.h with
raw device pointers and torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels. If libpalu.so is missing the
calls raise; there is no fallback.

Layouts (row-major): q [B, Hq, d]; h_k, h_v [B, G, L_cap, r] (int8 caches
with row scales s_k, s_v [B, G, L_cap] float32); b_k, b_v
[G, r, s*d]; seq_lens [B] int32; out [B, Hq, d] float32; x [B, d_model];
a_k, a_v [d_model, G*r] (or [G*r, d_model] with a_layout PALU_A_OUT_IN); pos
[B] int32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["PaluError", "AttnDesc", "AppendDesc", "PALU_F32", "PALU_BF16",
           "PALU_MODE_RECONSTRUCT", "PALU_MODE_ABSORBED", "PALU_MODE_FULL_RANK",
           "PALU_A_IN_OUT", "PALU_A_OUT_IN", "library",
           "library_path", "full_rank_attention",
           "palu_decode_attn_workspace", "palu_decode_attn_plan", "palu_decode_attn",
           "palu_decode_attn_noalloc",
           "palu_decode_attn_prepare", "palu_latent_append_prepare", "palu_decode_attn_i8",
           "decode_attention_i8",
           "palu_decode_attn_i4",
           "decode_attention_i4", "palu_latent_append_workspace",
           "palu_latent_append_i4_workspace", "palu_latent_append_i4", "latent_append_i4",
           "palu_latent_append_i8_workspace", "palu_latent_append_i8", "latent_append_i8", "palu_latent_append", "palu_profile_begin",
           "palu_profile_end", "attn_desc", "append_desc", "decode_attention", "latent_append",
           "EXPORTED_SYMBOLS"]

PALU_OK, PALU_ERR_NULL, PALU_ERR_SHAPE, PALU_ERR_UNSUPPORTED, PALU_ERR_WORKSPACE, \
    PALU_ERR_DEVICE = range(6)
PALU_F32, PALU_BF16 = 0, 1
PALU_MODE_RECONSTRUCT, PALU_MODE_ABSORBED, PALU_MODE_FULL_RANK = 0, 1, 2
PALU_A_IN_OUT, PALU_A_OUT_IN = 0, 1

EXPORTED_SYMBOLS = ("palu_decode_attn_workspace", "palu_decode_attn_plan", "palu_decode_attn",
                    "palu_decode_attn_noalloc",
                    "palu_decode_attn_prepare", "palu_decode_attn_i8", "palu_decode_attn_i4",
                    "palu_latent_append_workspace", "palu_latent_append",
                    "palu_latent_append_i8_workspace", "palu_latent_append_i8",
                    "palu_latent_append_i4_workspace", "palu_latent_append_i4",
                    "palu_latent_append_prepare", "palu_profile_begin", "palu_profile_end",
                    "palu_status_string", "palu_last_error")

_DIR = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("PALU_LIBRARY", os.path.join(_DIR, "libpalu.so"))


class PaluError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("scale", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("latent_out", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("prepared", ctypes.c_int32)]


class AppendDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("a_layout", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load libpalu.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libpalu.so not found at {path}: build it with "
                           f"`python -m rank_compressed_kv_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)
    lib.palu_decode_attn_workspace.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(sz)]
    lib.palu_decode_attn_plan.argtypes = [ctypes.POINTER(AttnDesc), i32p, i32p,
                                          ctypes.POINTER(ctypes.c_char_p)]
    lib.palu_decode_attn.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
    lib.palu_decode_attn_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp,
                                             vp, vp]
    lib.palu_decode_attn_prepare.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, sz, vp]
    for fn in ("palu_decode_attn_i8", "palu_decode_attn_i4"):
        getattr(lib, fn).argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, sz, vp]
    lib.palu_latent_append_workspace.argtypes = [ctypes.POINTER(AppendDesc), ctypes.POINTER(sz)]
    lib.palu_latent_append.argtypes = [ctypes.POINTER(AppendDesc), vp, vp, vp, vp, vp, vp, vp,
                                       sz, vp]
    for b in ("i8", "i4"):
        getattr(lib, f"palu_latent_append_{b}_workspace").argtypes = [
            ctypes.POINTER(AppendDesc), ctypes.POINTER(sz)]
        getattr(lib, f"palu_latent_append_{b}").argtypes = [
            ctypes.POINTER(AppendDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.palu_latent_append_prepare.argtypes = [
        ctypes.POINTER(AppendDesc), ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
        ctypes.POINTER(AttnDesc), vp, vp, vp, sz, vp]
    lib.palu_profile_begin.argtypes = [ctypes.c_int32]
    lib.palu_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), i32p]
    for fn in EXPORTED_SYMBOLS:
        if fn in ("palu_status_string", "palu_last_error"):
            continue
        getattr(lib, fn).restype = ctypes.c_int
    lib.palu_status_string.argtypes = [ctypes.c_int]
    lib.palu_status_string.restype = ctypes.c_char_p
    lib.palu_last_error.argtypes = []
    lib.palu_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != PALU_OK:
        lib = library()
        detail = (lib.palu_last_error() or b"").decode() or lib.palu_status_string(status).decode()
        raise PaluError(status, where, detail)


# ------------------------------------------------------------------ raw ABI ---

def palu_decode_attn_workspace(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(library().palu_decode_attn_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "palu_decode_attn_workspace")
    return int(n.value)


def palu_decode_attn_plan(desc: AttnDesc) -> Tuple[int, int, str]:
    ns, st, name = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_char_p()
    _check(library().palu_decode_attn_plan(ctypes.byref(desc), ctypes.byref(ns), ctypes.byref(st),
                                           ctypes.byref(name)), "palu_decode_attn_plan")
    return int(ns.value), int(st.value), name.value.decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PALU_F32
    if t.dtype == torch.bfloat16:
        return PALU_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    # the happy path costs a few attribute reads: a decode step makes two
    # calls, each checking up to nine tensors, and the checks run per call
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _desc_first(validate, desc, checks, *args):
    """Run the tensor checks; when one fails, let the library judge the
    descriptor first, so a bad descriptor is reported as the library's error
    (PaluError) rather than as a tensor mismatch it implies."""
    try:
        return checks(*args)
    except (TypeError, ValueError):
        validate(desc)
        raise


def _workspace_bytes(workspace) -> int:
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.numel() * workspace.element_size()


_TORCH_DTYPE = {PALU_F32: torch.float32, PALU_BF16: torch.bfloat16}


def _decode_checks(desc: AttnDesc, q, h_k, h_v, b_k, b_v, seq_lens, out) -> None:
    """Shapes, dtypes and devices of a decode call's tensors against desc."""
    _desc_first(palu_decode_attn_plan, desc, _decode_tensor_checks, desc, q, h_k, h_v, b_k,
                b_v, seq_lens, out)


def _decode_tensor_checks(desc: AttnDesc, q, h_k, h_v, b_k, b_v, seq_lens, out) -> None:
    B, Hq, Hkv, d = desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    G, r, L = desc.n_groups, desc.rank, desc.max_ctx
    dg = (Hkv // G) * d
    dt = _TORCH_DTYPE.get(desc.dtype)
    if dt is None:
        raise TypeError(f"unknown dtype code {desc.dtype}")
    _need(q, "q", (B, Hq, d), dt)
    _need(h_k, "h_k", (B, G, L, r), dt)
    _need(h_v, "h_v", (B, G, L, r), dt)
    full = desc.mode == PALU_MODE_FULL_RANK
    latent = not full and bool(desc.latent_out)
    if not full or b_k is not None:
        _need(b_k, "b_k", (G, r, dg), dt)
    if not (full or latent) or b_v is not None:
        _need(b_v, "b_v", (G, r, dg), dt)
    _need(out, "out", (B, Hq, r if latent else d), torch.float32)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", (B,), torch.int32)


def palu_decode_attn(desc: AttnDesc, q, h_k, h_v, b_k, b_v, seq_lens, out, workspace,
                     stream=None) -> None:
    """Enqueue one decode step. All tensors are checked against desc first."""
    _decode_checks(desc, q, h_k, h_v, b_k, b_v, seq_lens, out)
    nbytes = _workspace_bytes(workspace)
    _check(library().palu_decode_attn(
        ctypes.byref(desc), q.data_ptr(), h_k.data_ptr(), h_v.data_ptr(),
        None if b_k is None else b_k.data_ptr(), None if b_v is None else b_v.data_ptr(),
        None if seq_lens is None else seq_lens.data_ptr(), out.data_ptr(),
        workspace.data_ptr(), nbytes, _stream(stream)), "palu_decode_attn")


def palu_decode_attn_noalloc(desc: AttnDesc, q, h_k, h_v, b_k, b_v, seq_lens, out,
                             stream=None) -> None:
    """palu_decode_attn in the library's static scratch (no workspace; nothing
    is allocated). Calls overlapping in time on one GPU race."""
    _decode_checks(desc, q, h_k, h_v, b_k, b_v, seq_lens, out)
    _check(library().palu_decode_attn_noalloc(
        ctypes.byref(desc), q.data_ptr(), h_k.data_ptr(), h_v.data_ptr(),
        None if b_k is None else b_k.data_ptr(), None if b_v is None else b_v.data_ptr(),
        None if seq_lens is None else seq_lens.data_ptr(), out.data_ptr(), _stream(stream)),
        "palu_decode_attn_noalloc")


def _prepare_checks(desc: AttnDesc, q, b_k, workspace) -> int:
    """Shapes and dtypes of a prepare step's tensors; the workspace's bytes."""
    return _desc_first(palu_decode_attn_plan, desc, _prepare_tensor_checks, desc, q, b_k,
                       workspace)


def _prepare_tensor_checks(desc: AttnDesc, q, b_k, workspace) -> int:
    B, Hq, Hkv, d = desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    G, r = desc.n_groups, desc.rank
    dt = _TORCH_DTYPE.get(desc.dtype)
    if dt is None:
        raise TypeError(f"unknown dtype code {desc.dtype}")
    _need(q, "q", (B, Hq, d), dt)
    if desc.mode != PALU_MODE_FULL_RANK or b_k is not None:
        _need(b_k, "b_k", (G, r, (Hkv // G) * d), dt)
    return _workspace_bytes(workspace)


def palu_decode_attn_prepare(desc: AttnDesc, q, b_k, workspace, stream=None) -> None:
    """Form the decode call's query-side operands (q~, scaled q or B_k^T) in the
    workspace ahead of a call made with desc.prepared = 1."""
    nbytes = _prepare_checks(desc, q, b_k, workspace)
    _check(library().palu_decode_attn_prepare(
        ctypes.byref(desc), q.data_ptr(), None if b_k is None else b_k.data_ptr(),
        workspace.data_ptr(), nbytes, _stream(stream)), "palu_decode_attn_prepare")


def _decode_quant(bits: int, desc: AttnDesc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out,
                  workspace, stream) -> None:
    nbytes = _desc_first(palu_decode_attn_plan, desc, _quant_tensor_checks, bits, desc, q, h_k,
                         h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace)
    name = f"palu_decode_attn_i{bits}"
    _check(getattr(library(), name)(
        ctypes.byref(desc), q.data_ptr(), h_k.data_ptr(), h_v.data_ptr(), s_k.data_ptr(),
        s_v.data_ptr(), b_k.data_ptr(), None if b_v is None else b_v.data_ptr(),
        None if seq_lens is None else seq_lens.data_ptr(), out.data_ptr(),
        workspace.data_ptr(), nbytes, _stream(stream)), name)


def _quant_tensor_checks(bits: int, desc: AttnDesc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens,
                         out, workspace) -> int:
    B, Hq, Hkv, d = desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    G, r, L = desc.n_groups, desc.rank, desc.max_ctx
    dg = (Hkv // G) * d
    dt = _TORCH_DTYPE.get(desc.dtype)
    if dt is None:
        raise TypeError(f"unknown dtype code {desc.dtype}")
    latent = bool(desc.latent_out)
    cache = (B, G, L, r) if bits == 8 else (B, G, L, r // 2)
    ctype = torch.int8 if bits == 8 else torch.uint8
    _need(q, "q", (B, Hq, d), dt)
    _need(h_k, "h_k", cache, ctype)
    _need(h_v, "h_v", cache, ctype)
    _need(s_k, "s_k", (B, G, L), torch.float32)
    _need(s_v, "s_v", (B, G, L), torch.float32)
    _need(b_k, "b_k", (G, r, dg), dt)
    if not latent or b_v is not None:
        _need(b_v, "b_v", (G, r, dg), dt)
    _need(out, "out", (B, Hq, r if latent else d), torch.float32)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", (B,), torch.int32)
    return _workspace_bytes(workspace)


def palu_decode_attn_i8(desc: AttnDesc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out,
                        workspace, stream=None) -> None:
    """Enqueue one decode step over an int8 latent cache: h_k, h_v [B, G, L, r]
    int8 codes, s_k, s_v [B, G, L] float32 row scales."""
    _decode_quant(8, desc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace, stream)


def palu_decode_attn_i4(desc: AttnDesc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out,
                        workspace, stream=None) -> None:
    """Enqueue one decode step over an int4 latent cache: h_k, h_v [B, G, L, r/2]
    uint8 (two biased 4-bit codes a byte), s_k, s_v [B, G, L] float32."""
    _decode_quant(4, desc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace, stream)


def palu_latent_append_workspace(desc: AppendDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(library().palu_latent_append_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "palu_latent_append_workspace")
    return int(n.value)


def palu_latent_append(desc: AppendDesc, x, a_k, a_v, h_k, h_v, pos, workspace,
                       stream=None) -> None:
    nbytes = _append_checks(0, desc, x, a_k, a_v, h_k, h_v, None, None, pos, workspace)
    _check(library().palu_latent_append(
        ctypes.byref(desc), x.data_ptr(), a_k.data_ptr(), a_v.data_ptr(), h_k.data_ptr(),
        h_v.data_ptr(), pos.data_ptr(), workspace.data_ptr(), nbytes, _stream(stream)),
        "palu_latent_append")


def palu_latent_append_prepare(adesc: AppendDesc, qbits: int, x, a_k, a_v, h_k, h_v, s_k, s_v,
                               pos, append_ws, desc: AttnDesc, q, b_k, workspace,
                               stream=None) -> None:
    """The cache write qbits selects (0, 8, 4) and the decode call's query-side
    operands in one call (one launch when the absorption can ride in the
    append's); the decode call follows with desc.prepared = 1."""
    if qbits not in (0, 8, 4):
        raise ValueError(f"qbits must be 0, 8 or 4 (got {qbits})")
    abytes = _append_checks(qbits, adesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, append_ws)
    nbytes = _prepare_checks(desc, q, b_k, workspace)
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(library().palu_latent_append_prepare(
        ctypes.byref(adesc), qbits, x.data_ptr(), a_k.data_ptr(), a_v.data_ptr(),
        h_k.data_ptr(), h_v.data_ptr(), ptr(s_k), ptr(s_v), pos.data_ptr(),
        append_ws.data_ptr(), abytes, ctypes.byref(desc), q.data_ptr(), ptr(b_k),
        workspace.data_ptr(), nbytes, _stream(stream)), "palu_latent_append_prepare")


def palu_latent_append_i8_workspace(desc: AppendDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(library().palu_latent_append_i8_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "palu_latent_append_i8_workspace")
    return int(n.value)


def palu_latent_append_i4_workspace(desc: AppendDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(library().palu_latent_append_i4_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "palu_latent_append_i4_workspace")
    return int(n.value)


def _append_checks(bits: int, desc: AppendDesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos,
                   workspace) -> int:
    """Shapes and dtypes of an append's tensors (bits 0: dtype cache, 8 / 4:
    int8 / int4 codes with scales); the workspace's bytes."""
    validate = {0: palu_latent_append_workspace, 8: palu_latent_append_i8_workspace,
                4: palu_latent_append_i4_workspace}[bits]
    return _desc_first(validate, desc, _append_tensor_checks, bits, desc, x, a_k, a_v, h_k, h_v,
                       s_k, s_v, pos, workspace)


def _append_tensor_checks(bits: int, desc: AppendDesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos,
                          workspace) -> int:
    B, dm, G, r, L = desc.batch, desc.d_model, desc.n_groups, desc.rank, desc.max_ctx
    dt = _TORCH_DTYPE.get(desc.dtype)
    if dt is None:
        raise TypeError(f"unknown dtype code {desc.dtype}")
    _need(x, "x", (B, dm), dt)
    a_shape = (G * r, dm) if desc.a_layout == PALU_A_OUT_IN else (dm, G * r)
    _need(a_k, "a_k", a_shape, dt)
    _need(a_v, "a_v", a_shape, dt)
    if bits == 0:
        _need(h_k, "h_k", (B, G, L, r), dt)
        _need(h_v, "h_v", (B, G, L, r), dt)
    else:
        cache = (B, G, L, r) if bits == 8 else (B, G, L, r // 2)
        ctype = torch.int8 if bits == 8 else torch.uint8
        _need(h_k, "h_k", cache, ctype)
        _need(h_v, "h_v", cache, ctype)
        _need(s_k, "s_k", (B, G, L), torch.float32)
        _need(s_v, "s_v", (B, G, L), torch.float32)
    _need(pos, "pos", (B,), torch.int32)
    return _workspace_bytes(workspace)


def _append_quant(bits: int, desc: AppendDesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos,
                  workspace, stream) -> None:
    nbytes = _append_checks(bits, desc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace)
    name = f"palu_latent_append_i{bits}"
    _check(getattr(library(), name)(
        ctypes.byref(desc), x.data_ptr(), a_k.data_ptr(), a_v.data_ptr(), h_k.data_ptr(),
        h_v.data_ptr(), s_k.data_ptr(), s_v.data_ptr(), pos.data_ptr(), workspace.data_ptr(),
        nbytes, _stream(stream)), name)


def palu_latent_append_i8(desc: AppendDesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace,
                          stream=None) -> None:
    """Quantised cache write: h_k, h_v [B, G, L, r] int8, s_k, s_v [B, G, L] float32."""
    _append_quant(8, desc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream)


def palu_latent_append_i4(desc: AppendDesc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace,
                          stream=None) -> None:
    """Quantised cache write: h_k, h_v [B, G, L, r/2] uint8 (4-bit codes), s_k, s_v
    [B, G, L] float32."""
    _append_quant(4, desc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream)


def palu_profile_begin(max_records: int) -> None:
    _check(library().palu_profile_begin(int(max_records)), "palu_profile_begin")


def palu_profile_end() -> Tuple[float, int]:
    ms, n = ctypes.c_double(0), ctypes.c_int32(0)
    _check(library().palu_profile_end(ctypes.byref(ms), ctypes.byref(n)), "palu_profile_end")
    return float(ms.value), int(n.value)


# ------------------------------------------------------------- convenience ---

def attn_desc(*, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_groups: int,
              rank: int, max_ctx: int, dtype: int, mode: str = "reconstruct",
              rope_theta: float = 0.0, scale: float = 0.0, split_tokens: int = 0,
              latent_out: bool = False, hadamard: bool = False,
              prepared: bool = False) -> AttnDesc:
    modes = {"reconstruct": PALU_MODE_RECONSTRUCT, "absorbed": PALU_MODE_ABSORBED,
             "full_rank": PALU_MODE_FULL_RANK}
    if mode not in modes:
        raise ValueError(f"mode must be one of {sorted(modes)}")
    return AttnDesc(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                    n_groups=n_groups, rank=rank, max_ctx=max_ctx, dtype=dtype, mode=modes[mode],
                    split_tokens=split_tokens, scale=scale, rope_theta=rope_theta,
                    latent_out=1 if latent_out else 0, hadamard=1 if hadamard else 0,
                    prepared=1 if prepared else 0)


def append_desc(*, batch: int, d_model: int, n_groups: int, rank: int, max_ctx: int,
                dtype: int, hadamard: bool = False, a_layout: int = 0) -> AppendDesc:
    """a_layout PALU_A_IN_OUT (0): a_k, a_v [d_model, G*r]; PALU_A_OUT_IN (1):
    [G*r, d_model], the torch.nn.Linear weight layout."""
    return AppendDesc(batch=batch, d_model=d_model, n_groups=n_groups, rank=rank,
                      max_ctx=max_ctx, dtype=dtype, hadamard=1 if hadamard else 0,
                      a_layout=a_layout)


def decode_attention(q, h_k, h_v, b_k, b_v, seq_lens=None, *, n_kv_heads: int,
                     mode: str = "reconstruct", rope_theta: float = 0.0, scale: float = 0.0,
                     split_tokens: int = 0, latent_out: bool = False, out=None,
                     workspace=None, stream=None):
    """Shapes are read from the tensors; n_kv_heads fixes the head layout.
    With latent_out the result is u* [B, Hq, r] and b_v may be None.
    Allocates out and the workspace with torch when they are not given."""
    B, Hq, d = q.shape
    _, G, L, r = h_k.shape
    desc = attn_desc(batch=B, n_q_heads=Hq, n_kv_heads=n_kv_heads, head_dim=d, n_groups=G,
                     rank=r, max_ctx=L, dtype=_dt(q), mode=mode, rope_theta=rope_theta,
                     scale=scale, split_tokens=split_tokens, latent_out=latent_out)
    if out is None:
        out = torch.empty((B, Hq, r if latent_out else d), dtype=torch.float32,
                          device=q.device)
    if workspace is None:
        workspace = torch.empty(palu_decode_attn_workspace(desc), dtype=torch.uint8,
                                device=q.device)
    palu_decode_attn(desc, q, h_k, h_v, b_k, b_v, seq_lens, out, workspace, stream)
    return out


def _decode_attention_quant(bits, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, n_kv_heads,
                            scale, split_tokens, latent_out, hadamard, out, workspace, stream):
    B, Hq, d = q.shape
    _, G, L, rr = h_k.shape
    r = rr if bits == 8 else 2 * rr
    desc = attn_desc(batch=B, n_q_heads=Hq, n_kv_heads=n_kv_heads, head_dim=d, n_groups=G,
                     rank=r, max_ctx=L, dtype=_dt(q), mode="absorbed", scale=scale,
                     split_tokens=split_tokens, latent_out=latent_out, hadamard=hadamard)
    if out is None:
        out = torch.empty((B, Hq, r if latent_out else d), dtype=torch.float32,
                          device=q.device)
    if workspace is None:
        workspace = torch.empty(palu_decode_attn_workspace(desc), dtype=torch.uint8,
                                device=q.device)
    _decode_quant(bits, desc, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace, stream)
    return out


def decode_attention_i8(q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens=None, *, n_kv_heads: int,
                        scale: float = 0.0, split_tokens: int = 0, latent_out: bool = False,
                        hadamard: bool = False, out=None, workspace=None, stream=None):
    """Absorbed-mode decode over int8 latents (codes h_k, h_v with row scales
    s_k, s_v). Allocates out and the workspace with torch when not given."""
    return _decode_attention_quant(8, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, n_kv_heads,
                                   scale, split_tokens, latent_out, hadamard, out, workspace,
                                   stream)


def decode_attention_i4(q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens=None, *, n_kv_heads: int,
                        scale: float = 0.0, split_tokens: int = 0, latent_out: bool = False,
                        hadamard: bool = False, out=None, workspace=None, stream=None):
    """Absorbed-mode decode over int4 latents (h_k, h_v [B, G, L, r/2] uint8 in
    the tiled nibble order, row scales s_k, s_v). Allocates out and the
    workspace with torch when not given."""
    return _decode_attention_quant(4, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, n_kv_heads,
                                   scale, split_tokens, latent_out, hadamard, out, workspace,
                                   stream)


def full_rank_attention(q, k, v, seq_lens=None, *, scale: float = 0.0, split_tokens: int = 0,
                        out=None, workspace=None, stream=None):
    """The uncompressed baseline: k, v [B, Hkv, L, d] hold the full (already
    rotated) keys and values. Allocates out and the workspace when not given."""
    B, Hq, d = q.shape
    _, Hkv, L, dk = k.shape
    desc = attn_desc(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, n_groups=Hkv,
                     rank=dk, max_ctx=L, dtype=_dt(q), mode="full_rank", scale=scale,
                     split_tokens=split_tokens)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(palu_decode_attn_workspace(desc), dtype=torch.uint8,
                                device=q.device)
    palu_decode_attn(desc, q, k, v, None, None, seq_lens, out, workspace, stream)
    return out


def latent_append(x, a_k, a_v, h_k, h_v, pos, workspace=None, stream=None, *,
                  a_layout: int = 0) -> None:
    """Allocates the workspace with torch when it is not given. a_layout
    PALU_A_OUT_IN takes a_k, a_v as [G*r, d_model]."""
    B, dm = x.shape
    _, G, L, r = h_k.shape
    desc = append_desc(batch=B, d_model=dm, n_groups=G, rank=r, max_ctx=L, dtype=_dt(x),
                       a_layout=a_layout)
    if workspace is None:
        workspace = torch.zeros(palu_latent_append_workspace(desc), dtype=torch.uint8,
                                device=x.device)
    palu_latent_append(desc, x, a_k, a_v, h_k, h_v, pos, workspace, stream)


def _latent_append_quant(bits, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream,
                         hadamard) -> None:
    B, dm = x.shape
    _, G, L, rr = h_k.shape
    r = rr if bits == 8 else 2 * rr
    desc = append_desc(batch=B, d_model=dm, n_groups=G, rank=r, max_ctx=L, dtype=_dt(x),
                       hadamard=hadamard)
    if workspace is None:
        need = (palu_latent_append_i8_workspace if bits == 8
                else palu_latent_append_i4_workspace)(desc)
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    _append_quant(bits, desc, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream)


def latent_append_i8(x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace=None, stream=None, *,
                     hadamard: bool = False) -> None:
    """Quantised cache write into an int8 cache (rows rotated by the Hadamard
    matrix first with hadamard=True). Allocates the (zeroed) workspace with
    torch when it is not given."""
    _latent_append_quant(8, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream, hadamard)


def latent_append_i4(x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace=None, stream=None, *,
                     hadamard: bool = False) -> None:
    """Quantised cache write into an int4 cache (h_k, h_v [B, G, L, r/2] uint8).
    Allocates the (zeroed) workspace with torch when it is not given."""
    _latent_append_quant(4, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, stream, hadamard)
