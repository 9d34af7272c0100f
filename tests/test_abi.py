"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import rank_compressed_kv_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "palu.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.library_path()):
        from rank_compressed_kv_amd import build
        build.build()
    return P.library()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(palu_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert set(declared) == set(P.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def _desc(**kw):
    base = dict(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, n_groups=2, rank=256,
                max_ctx=32768, dtype=P.PALU_BF16, mode="absorbed")
    base.update(kw)
    return P.attn_desc(**base)


BAD = [
    (dict(batch=0), P.PALU_ERR_SHAPE),
    (dict(n_q_heads=30), P.PALU_ERR_SHAPE),
    (dict(n_groups=3), P.PALU_ERR_SHAPE),
    (dict(head_dim=127), P.PALU_ERR_SHAPE),
    (dict(head_dim=258), P.PALU_ERR_SHAPE),
    (dict(rank=513), P.PALU_ERR_SHAPE),
    (dict(rank=0), P.PALU_ERR_SHAPE),
    (dict(max_ctx=0), P.PALU_ERR_SHAPE),
    (dict(split_tokens=100), P.PALU_ERR_SHAPE),
    (dict(split_tokens=-64), P.PALU_ERR_SHAPE),
    (dict(dtype=7), P.PALU_ERR_UNSUPPORTED),
    (dict(rope_theta=5e5), P.PALU_ERR_UNSUPPORTED),          # absorbed + RoPE
    (dict(mode="reconstruct", rope_theta=-1.0), P.PALU_ERR_UNSUPPORTED),
    (dict(mode="reconstruct", rope_theta=float("nan")), P.PALU_ERR_UNSUPPORTED),
    # the uncompressed baseline: one group per KV head, rank = head_dim, no RoPE
    (dict(mode="full_rank", n_groups=8, rank=128, rope_theta=5e5), P.PALU_ERR_UNSUPPORTED),
    (dict(mode="full_rank", n_groups=2, rank=128), P.PALU_ERR_SHAPE),
    (dict(mode="full_rank", n_groups=8, rank=256), P.PALU_ERR_SHAPE),
]


def test_latent_output_needs_no_bv(lib):
    """latent_out: b_v may be NULL (the check moves on to the workspace); without
    it a NULL b_v is an error. b_k stays required."""
    fake = ctypes.c_void_p(0x1000)
    d = _desc(latent_out=True)
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, None, None, fake,
                                fake, 16, None) == P.PALU_ERR_WORKSPACE
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake,
                                fake, 1 << 40, None) == P.PALU_ERR_NULL
    d = _desc()
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, None, None, fake,
                                fake, 1 << 40, None) == P.PALU_ERR_NULL


def test_full_rank_mode_needs_no_factors(lib):
    """FULL_RANK accepts NULL b_k, b_v (it never reads them) but not a NULL cache."""
    d = _desc(mode="full_rank", n_groups=8, rank=128)
    n = ctypes.c_size_t(0)
    assert lib.palu_decode_attn_workspace(ctypes.byref(d), ctypes.byref(n)) == P.PALU_OK
    heads = 8 * 32
    assert n.value >= heads * 128 * 4          # the pre-scaled queries
    _, _, kname = P.palu_decode_attn_plan(d)
    assert kname == "split_absorbed_mfma_kernel"
    fake = ctypes.c_void_p(0x1000)
    assert lib.palu_decode_attn(ctypes.byref(d), fake, None, fake, None, None, None, fake,
                                fake, 1 << 40, None) == P.PALU_ERR_NULL
    # too small a workspace is caught before anything is launched
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, None, None, None, fake,
                                fake, 16, None) == P.PALU_ERR_WORKSPACE


def test_prepare_validation(lib):
    """The prepare step checks the descriptor (prepared must be 0 or 1), its
    pointers (b_k may be NULL only in FULL_RANK mode) and the workspace before
    launching anything."""
    fake = ctypes.c_void_p(0x1000)
    d = _desc(prepared=True)
    d.prepared = 2
    assert lib.palu_decode_attn_prepare(ctypes.byref(d), fake, fake, fake, 1 << 40,
                                        None) == P.PALU_ERR_UNSUPPORTED
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake,
                                fake, 1 << 40, None) == P.PALU_ERR_UNSUPPORTED
    d.prepared = 1
    for mode, kw in (("absorbed", {}), ("reconstruct", dict(rope_theta=5e5))):
        d = _desc(mode=mode, **kw)
        assert lib.palu_decode_attn_prepare(ctypes.byref(d), None, fake, fake, 1 << 40,
                                            None) == P.PALU_ERR_NULL
        assert lib.palu_decode_attn_prepare(ctypes.byref(d), fake, None, fake, 1 << 40,
                                            None) == P.PALU_ERR_NULL
        assert lib.palu_decode_attn_prepare(ctypes.byref(d), fake, fake, None, 1 << 40,
                                            None) == P.PALU_ERR_NULL
        need = P.palu_decode_attn_workspace(d)
        assert lib.palu_decode_attn_prepare(ctypes.byref(d), fake, fake, fake, need - 1,
                                            None) == P.PALU_ERR_WORKSPACE
    d = _desc(mode="full_rank", n_groups=8, rank=128)
    assert lib.palu_decode_attn_prepare(ctypes.byref(d), fake, None, fake, 16,
                                        None) == P.PALU_ERR_WORKSPACE


def _quant(lib, bits, d, *ptrs, nbytes=1 << 40):
    fake = ctypes.c_void_p(0x1000)
    q, hk, hv, sk, sv, bk, bv, out, ws = [fake if p is True else p for p in ptrs]
    fn = lib.palu_decode_attn_i8 if bits == 8 else lib.palu_decode_attn_i4
    return fn(ctypes.byref(d), q, hk, hv, sk, sv, bk, bv, None, out, ws, nbytes, None)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("kw", [dict(mode="reconstruct", rope_theta=5e5),
                                dict(mode="full_rank", n_groups=8, rank=128),
                                dict(dtype=P.PALU_F32), dict(rank=32), dict(rank=512),
                                dict(rank=96)])
def test_quant_decode_unsupported_combinations(lib, kw, bits):
    """int8 / int4 latents are provided for ABSORBED, BF16, rank 64/128/256 only."""
    assert _quant(lib, bits, _desc(**kw), *([True] * 9)) == P.PALU_ERR_UNSUPPORTED
    assert f"int{bits}".encode() in lib.palu_last_error()


@pytest.mark.parametrize("bits", [8, 4])
def test_quant_decode_validation(lib, bits):
    """Descriptor errors come first (the tiled caches need max_ctx % 32 == 0),
    then missing pointers, 16-byte alignment, then the workspace (same size as
    palu_decode_attn's)."""

    assert _quant(lib, bits, _desc(batch=0), *([True] * 9)) == P.PALU_ERR_SHAPE
    assert _quant(lib, bits, _desc(max_ctx=1000), *([True] * 9)) == P.PALU_ERR_SHAPE
    odd = ctypes.c_void_p(0x1008)
    for i in (1, 2, 3, 4):                   # h_k, h_v, s_k, s_v
        ptrs = [True] * 9
        ptrs[i] = odd
        assert _quant(lib, bits, _desc(), *ptrs) == P.PALU_ERR_SHAPE, i
    d = _desc(rank=128)
    for i in range(9):                       # every pointer is needed here
        ptrs = [True] * 9
        ptrs[i] = None
        assert _quant(lib, bits, d, *ptrs, nbytes=16) == P.PALU_ERR_NULL, i
    # latent_out: b_v may be NULL
    d = _desc(rank=128, latent_out=True)
    ptrs = [True] * 9
    ptrs[6] = None
    assert _quant(lib, bits, d, *ptrs, nbytes=16) == P.PALU_ERR_WORKSPACE
    need = P.palu_decode_attn_workspace(d)
    assert _quant(lib, bits, d, *([True] * 9), nbytes=need - 1) == P.PALU_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", BAD)
def test_descriptor_validation(lib, kw, status):
    d = _desc(**kw)
    n = ctypes.c_size_t(0)
    assert lib.palu_decode_attn_workspace(ctypes.byref(d), ctypes.byref(n)) == status
    assert lib.palu_last_error()
    # the decode call itself rejects the same descriptor before touching the device
    fake = ctypes.c_void_p(0x1000)
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake,
                                fake, 1 << 40, None) == status


def test_bad_mode(lib):
    d = _desc()
    d.mode = 5
    assert lib.palu_decode_attn_plan(ctypes.byref(d), None, None, None) == P.PALU_ERR_UNSUPPORTED


def test_null_pointers_and_workspace(lib):
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    assert lib.palu_decode_attn(None, fake, fake, fake, fake, fake, None, fake, fake, 1 << 40,
                                None) == P.PALU_ERR_NULL
    for i in range(7):
        ptrs = [fake] * 7
        ptrs[i] = None
        q, hk, hv, bk, bv, out, ws = ptrs
        assert lib.palu_decode_attn(ctypes.byref(d), q, hk, hv, bk, bv, None, out, ws, 1 << 40,
                                    None) == P.PALU_ERR_NULL
    need = P.palu_decode_attn_workspace(d)
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake,
                                need - 1, None) == P.PALU_ERR_WORKSPACE
    assert b"needs" in lib.palu_last_error()


def test_workspace_covers_partials_and_plan_covers_context(lib):
    for mode in ("absorbed", "reconstruct"):
        for st in (0, 64, 512, 4096):
            d = _desc(mode=mode, split_tokens=st)
            ns, tok, name = P.palu_decode_attn_plan(d)
            assert tok % 64 == 0 and ns * tok >= d.max_ctx > (ns - 1) * tok
            if st:
                assert tok == st
            heads = d.batch * d.n_q_heads
            need = P.palu_decode_attn_workspace(d)
            assert need >= heads * ns * (d.rank + 2) * 4
            if mode == "absorbed":
                assert need >= heads * ns * (d.rank + 2) * 4 + heads * d.rank * 4
            assert isinstance(name, str) and name


def test_append_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    good = P.append_desc(batch=8, d_model=4096, n_groups=2, rank=256, max_ctx=32768,
                         dtype=P.PALU_BF16)
    bad = [(dict(batch=0), P.PALU_ERR_SHAPE), (dict(rank=600), P.PALU_ERR_SHAPE),
           (dict(n_groups=1, rank=12), P.PALU_ERR_SHAPE),
           (dict(d_model=70000), P.PALU_ERR_SHAPE), (dict(dtype=3), P.PALU_ERR_UNSUPPORTED)]
    big = 1 << 40
    for kw, status in bad:
        d = P.AppendDesc(**{**{f: getattr(good, f) for f, _ in P.AppendDesc._fields_}, **kw})
        assert lib.palu_latent_append(ctypes.byref(d), fake, fake, fake, fake, fake, fake,
                                      fake, big, None) == status
        n = ctypes.c_size_t(0)
        assert lib.palu_latent_append_workspace(ctypes.byref(d), ctypes.byref(n)) == status
    for i in range(7):
        ptrs = [fake] * 7
        ptrs[i] = None
        assert lib.palu_latent_append(ctypes.byref(good), *ptrs, big, None) == P.PALU_ERR_NULL
    assert lib.palu_latent_append(None, fake, fake, fake, fake, fake, fake, fake, big,
                                  None) == P.PALU_ERR_NULL
    need = P.palu_latent_append_workspace(good)
    # 256 bytes of arrival counters (8 column blocks of 128), then the partials
    # of 128-row slices x batch x (k and v columns)
    assert need == 256 + 32 * 8 * 1024 * 4
    assert lib.palu_latent_append(ctypes.byref(good), fake, fake, fake, fake, fake, fake, fake,
                                  need - 1, None) == P.PALU_ERR_WORKSPACE
    misaligned = ctypes.c_void_p(0x1008)
    assert lib.palu_latent_append(ctypes.byref(good), fake, fake, fake, fake, fake, fake,
                                  misaligned, need, None) == P.PALU_ERR_WORKSPACE


def test_append_layout_validation(lib):
    """a_layout: 0 or 1; the transposed projection needs d_model % 8 == 0 and
    no workspace (size 0), and is not offered for the quantised caches. Every
    call here is rejected, so nothing is launched on the fake pointers."""
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    cols = P.append_desc(batch=8, d_model=4096, n_groups=2, rank=256, max_ctx=32768,
                         dtype=P.PALU_BF16, a_layout=P.PALU_A_OUT_IN)
    assert P.palu_latent_append_workspace(cols) == 0
    for kw, status in ((dict(a_layout=2), P.PALU_ERR_UNSUPPORTED),
                       (dict(a_layout=-1), P.PALU_ERR_UNSUPPORTED),
                       (dict(d_model=4100), P.PALU_ERR_SHAPE)):
        d = P.AppendDesc(**{**{f: getattr(cols, f) for f, _ in P.AppendDesc._fields_}, **kw})
        n = ctypes.c_size_t(0)
        assert lib.palu_latent_append_workspace(ctypes.byref(d), ctypes.byref(n)) == status
        assert lib.palu_latent_append(ctypes.byref(d), fake, fake, fake, fake, fake, fake,
                                      fake, big, None) == status
    # the row-major form still accepts d_model 4100
    rows = P.AppendDesc(**{**{f: getattr(cols, f) for f, _ in P.AppendDesc._fields_},
                           "d_model": 4100, "a_layout": P.PALU_A_IN_OUT})
    assert P.palu_latent_append_workspace(rows) > 0
    for i in range(6):                            # x, a_k, a_v, h_k, h_v, pos
        ptrs = [fake] * 6
        ptrs[i] = None
        assert lib.palu_latent_append(ctypes.byref(cols), *ptrs, None, 0,
                                      None) == P.PALU_ERR_NULL
    for bits in (8, 4):
        n = ctypes.c_size_t(0)
        assert getattr(lib, f"palu_latent_append_i{bits}_workspace")(
            ctypes.byref(cols), ctypes.byref(n)) == P.PALU_ERR_UNSUPPORTED
        assert getattr(lib, f"palu_latent_append_i{bits}")(
            ctypes.byref(cols), fake, fake, fake, fake, fake, fake, fake, fake, fake, big,
            None) == P.PALU_ERR_UNSUPPORTED


def test_append_prepare_validation(lib):
    """The combined step checks both calls' arguments before launching
    anything: the append's (per qbits) and the prepare step's. Every call here
    is rejected, so nothing is launched on the fake pointers."""
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    ad = P.append_desc(batch=8, d_model=4096, n_groups=2, rank=256, max_ctx=32768,
                       dtype=P.PALU_BF16)
    d = _desc()

    def call(qbits=0, ad_=ad, d_=d, a=None, b=None):
        a = [fake] * 9 if a is None else a       # x, a_k, a_v, h_k, h_v, s_k, s_v, pos, ws
        b = [fake] * 3 if b is None else b       # q, b_k, workspace
        return lib.palu_latent_append_prepare(
            None if ad_ is None else ctypes.byref(ad_), qbits, *a[:8], a[8], big,
            None if d_ is None else ctypes.byref(d_), b[0], b[1], b[2], big, None)

    assert call(qbits=3) == P.PALU_ERR_UNSUPPORTED
    assert call(ad_=None) == P.PALU_ERR_NULL
    assert call(d_=None) == P.PALU_ERR_NULL
    for i in (0, 1, 2, 3, 4, 7, 8):              # every append pointer but the scales
        a = [fake] * 9
        a[i] = None
        assert call(a=a) == P.PALU_ERR_NULL
    for bits in (8, 4):
        for i in (5, 6):                          # the scales, for a quantised cache
            a = [fake] * 9
            a[i] = None
            assert call(qbits=bits, a=a) == P.PALU_ERR_NULL
    for i in range(3):
        b = [fake] * 3
        b[i] = None
        assert call(b=b) == P.PALU_ERR_NULL
    bad = P.AppendDesc(**{**{f: getattr(ad, f) for f, _ in P.AppendDesc._fields_}, "hadamard": 1})
    assert call(ad_=bad) == P.PALU_ERR_UNSUPPORTED   # a dtype cache has no Hadamard form
    worse = _desc(head_dim=3)
    assert call(d_=worse) == P.PALU_ERR_SHAPE
    need = P.palu_decode_attn_workspace(d)
    assert lib.palu_latent_append_prepare(
        ctypes.byref(ad), 0, *([fake] * 8), fake, big, ctypes.byref(d), fake, fake, fake,
        need - 1, None) == P.PALU_ERR_WORKSPACE
    aneed = P.palu_latent_append_workspace(ad)
    assert lib.palu_latent_append_prepare(
        ctypes.byref(ad), 0, *([fake] * 8), fake, aneed - 1, ctypes.byref(d), fake, fake, fake,
        big, None) == P.PALU_ERR_WORKSPACE
    # the two workspaces may not share a byte (checked before any launch):
    # the decode workspace starting inside the append's, or the append's
    # starting inside the decode one's
    a0 = 1 << 32
    for w0 in (a0 + aneed - 256, a0 - need + 256, a0):
        assert lib.palu_latent_append_prepare(
            ctypes.byref(ad), 0, *([fake] * 8), ctypes.c_void_p(a0), aneed, ctypes.byref(d),
            fake, fake, ctypes.c_void_p(w0), need, None) == P.PALU_ERR_WORKSPACE, hex(w0)
    assert b"overlap" in lib.palu_last_error()


@pytest.mark.parametrize("bits", [8, 4])
def test_append_quant_validation(lib, bits):
    """The quantised cache write: the append checks, rank 64/128/256, NULL
    scales, 4-byte aligned caches, and the dtype append's workspace (the same
    for both widths)."""
    fake = ctypes.c_void_p(0x1000)
    good = P.append_desc(batch=8, d_model=4096, n_groups=2, rank=256, max_ctx=32768,
                         dtype=P.PALU_BF16)
    big = 1 << 40

    def call(d, *ptrs, nbytes=big):
        ptrs = [fake if p is True else p for p in ptrs]
        fn = lib.palu_latent_append_i8 if bits == 8 else lib.palu_latent_append_i4
        return fn(ctypes.byref(d), *ptrs, nbytes, None)

    def workspace_call(d, n):
        fn = (lib.palu_latent_append_i8_workspace if bits == 8
              else lib.palu_latent_append_i4_workspace)
        return fn(ctypes.byref(d), ctypes.byref(n))

    bad = [(dict(batch=0), P.PALU_ERR_SHAPE), (dict(rank=600), P.PALU_ERR_SHAPE),
           (dict(n_groups=4, rank=6), P.PALU_ERR_UNSUPPORTED),  # the tiled cache: r 64/128/256
           (dict(n_groups=4, rank=96), P.PALU_ERR_UNSUPPORTED),
           (dict(max_ctx=1000), P.PALU_ERR_SHAPE),              # whole 32-token blocks
           (dict(dtype=3), P.PALU_ERR_UNSUPPORTED)]
    for kw, status in bad:
        d = P.AppendDesc(**{**{f: getattr(good, f) for f, _ in P.AppendDesc._fields_}, **kw})
        assert call(d, *([True] * 9)) == status
        n = ctypes.c_size_t(0)
        assert workspace_call(d, n) == status
    for i in range(9):
        ptrs = [True] * 9
        ptrs[i] = None
        assert call(good, *ptrs) == P.PALU_ERR_NULL, i
    need = (P.palu_latent_append_i8_workspace if bits == 8
            else P.palu_latent_append_i4_workspace)(good)
    # the same areas as the dtype append: column-block counters (256 B),
    # then the partials
    assert need == 256 + 32 * 8 * 1024 * 4
    assert call(good, *([True] * 9), nbytes=need - 1) == P.PALU_ERR_WORKSPACE
    odd = ctypes.c_void_p(0x1002)
    assert call(good, True, True, True, odd, True, True, True, True, True) == P.PALU_ERR_SHAPE
    assert call(good, *([True] * 8), ctypes.c_void_p(0x1008)) == P.PALU_ERR_WORKSPACE


@pytest.mark.parametrize("bits", [8, 4])
def test_hadamard_flag_is_for_quantised_caches_only(lib, bits):
    """The rotated-cache flag is refused by the bf16 calls, accepted by the
    int8 and int4 ones (which then fail on the fake workspace size), and must
    be 0/1."""
    append_q = lib.palu_latent_append_i8 if bits == 8 else lib.palu_latent_append_i4
    fake = ctypes.c_void_p(0x1000)
    d = _desc(rank=128, hadamard=True)
    assert lib.palu_decode_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake,
                                fake, 1 << 40, None) == P.PALU_ERR_UNSUPPORTED
    assert b"int8" in lib.palu_last_error()
    assert _quant(lib, bits, d, *([True] * 9), nbytes=16) == P.PALU_ERR_WORKSPACE
    d.hadamard = 2
    assert _quant(lib, bits, d, *([True] * 9)) == P.PALU_ERR_UNSUPPORTED
    a = P.append_desc(batch=2, d_model=256, n_groups=2, rank=64, max_ctx=64,
                      dtype=P.PALU_BF16, hadamard=True)
    assert lib.palu_latent_append(ctypes.byref(a), fake, fake, fake, fake, fake, fake, fake,
                                  1 << 40, None) == P.PALU_ERR_UNSUPPORTED
    assert append_q(ctypes.byref(a), *([fake] * 9), 16, None) == P.PALU_ERR_WORKSPACE
    a.hadamard = -1
    assert append_q(ctypes.byref(a), *([fake] * 9), 1 << 40, None) == P.PALU_ERR_UNSUPPORTED


def test_only_the_c_abi_is_exported(lib):
    """Every function the library exports is one the header declares."""
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", P.library_path()], capture_output=True,
                         text=True, check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]}
    assert funcs == set(_header_functions())


def test_profile_calls_validate(lib):
    assert lib.palu_profile_end(None, None) == P.PALU_ERR_UNSUPPORTED
    assert lib.palu_profile_begin(0) == P.PALU_ERR_SHAPE


def test_status_strings(lib):
    for s in range(6):
        assert lib.palu_status_string(s)
    assert lib.palu_status_string(42) == b"unknown status"


def test_binding_rejects_cpu_tensors():
    import torch
    d = _desc(batch=1, max_ctx=64)
    q = torch.zeros(1, 32, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        P.palu_decode_attn(d, q, q, q, q, q, None, q, q)


def test_noalloc_validation(lib):
    """The entry point without a workspace checks everything on the host
    first: the descriptor, the operand pointers, prepared / hadamard, and the
    scratch the call needs against the static scratch's 32 MiB. Every call
    here is rejected before any HIP call, so nothing is launched."""
    fake = ctypes.c_void_p(0x1000)
    ops = [fake] * 5 + [None, fake]          # q, h_k, h_v, b_k, b_v, seq_lens, out

    def call(d, ops_=ops):
        return lib.palu_decode_attn_noalloc(ctypes.byref(d), *ops_, None)

    assert lib.palu_decode_attn_noalloc(None, *ops, None) == P.PALU_ERR_NULL
    assert call(_desc(head_dim=127)) == P.PALU_ERR_SHAPE
    for i in (0, 1, 2, 3, 4, 6):
        o = list(ops)
        o[i] = None
        assert call(_desc(), o) == P.PALU_ERR_NULL, i
    assert call(_desc(prepared=True)) == P.PALU_ERR_UNSUPPORTED
    assert call(_desc(hadamard=True)) == P.PALU_ERR_UNSUPPORTED
    # far beyond 32 MiB of split partials: rejected with the figure it needs
    big = _desc(batch=256)
    need = P.palu_decode_attn_workspace(big)
    assert need > 32 << 20
    assert call(big) == P.PALU_ERR_WORKSPACE
    assert str(need).encode() in lib.palu_last_error()
