"""Plant plausible mistakes in the oracle (on the CPU, by rewriting its source in a
scratch namespace) and check that the pins catch every one of them."""
import inspect
import json
import os
import types

import numpy as np
import pytest

from oracle import palu_oracle as O
import tests.test_oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")

MUTANTS = {
    "rope_sign": ("apply_rope", "[c * x - s * y, s * x + c * y]", "[c * x + s * y, -s * x + c * y]"),
    "rope_interleaved": ("apply_rope", "x, y = k[:, :half], k[:, half:]",
                         "x, y = k[:, 0::2], k[:, 1::2]"),
    "rope_freq_exponent": ("rope_angles", "-2.0 * i / head_dim", "-1.0 * i / head_dim"),
    "rope_positions_from_1": ("decode_attention", "pos = np.arange(n)", "pos = np.arange(1, n + 1)"),
    "no_scale": ("decode_attention", "out[b, h] = attend(to_f64(q[b, h]), Kj, Vj, scale)",
                 "out[b, h] = attend(to_f64(q[b, h]), Kj, Vj, 1.0)"),
    "gqa_modulo": ("decode_attention", "j = h // gqa", "j = h % (G * s)"),
    "head_columns_strided": ("decode_attention", "Kj = apply_rope(Kg[:, jl * d:(jl + 1) * d]",
                             "Kj = apply_rope(Kg[:, jl::s]"),
    "value_uses_keys": ("decode_attention", "Vj = Vg[:, jl * d:(jl + 1) * d]",
                        "Vj = Kg[:, jl * d:(jl + 1) * d]"),
    "full_rank_gqa_modulo": ("full_rank_attention", "j = h // gqa", "j = h % Hkv"),
    "full_rank_value_uses_keys": ("full_rank_attention", "to_f64(k[b, j, :n]), to_f64(v[b, j, :n])",
                                  "to_f64(k[b, j, :n]), to_f64(k[b, j, :n])"),
    "full_rank_len_off_by_one": ("full_rank_attention", "n = int(lens[b])",
                                 "n = max(0, int(lens[b]) - 1)"),
    "latents_value_uses_keys": ("decode_value_latents", "Hv = to_f64(h_v[b, g, :n])",
                                "Hv = to_f64(h_k[b, g, :n])"),
    "latents_gqa_modulo": ("decode_value_latents", "jl = h // gqa - g * s", "jl = h % s"),
    "quant_floor": ("quantize_rows_i8", "np.clip(np.rint(prod)", "np.clip(np.floor(prod)"),
    "quant_128_steps": ("quantize_rows_i8", "np.float32(127.0) / safe", "np.float32(128.0) / safe"),
    "quant_ties_away": ("quantize_rows_i8", "np.clip(np.rint(prod)",
                        "np.clip(np.sign(prod) * np.floor(np.abs(prod) + 0.5)"),
    "quant_column_amax": ("quantize_rows_i8", "amax = np.max(np.abs(h), axis=-1)",
                          "amax = np.broadcast_to(np.max(np.abs(h)), h.shape[:-1])"),
    "quant4_8_steps": ("quantize_rows_i4", "np.float32(7.0) / safe", "np.float32(8.0) / safe"),
    "quant4_floor": ("quantize_rows_i4", "np.clip(np.rint(prod), -7, 7)",
                     "np.clip(np.floor(prod), -7, 7)"),
    "quant4_clamp_8": ("quantize_rows_i4", "np.clip(np.rint(prod), -7, 7)",
                       "np.clip(np.rint(prod * np.float32(1.1)), -8, 7)"),
    "hadamard_block_sign": ("hadamard", "h = np.block([[h, h], [h, -h]])",
                            "h = np.block([[h, h], [-h, h]])"),
    "hadamard_no_rescale": ("dequantize_rows_i8_hadamard", "@ hadamard(r) / r", "@ hadamard(r)"),
    "hadamard_quantise_first": ("append_rows_i8_hadamard", "rot = h @ hadamard(h.shape[-1])",
                                "rot = h"),
    "softmax_unnormalised": ("softmax", "return e / np.sum(e, axis=-1, keepdims=True)", "return e"),
    "reconstruct_transposed": ("reconstruct", "return to_f64(h) @ to_f64(b)",
                               "return to_f64(h) @ to_f64(b)[::-1]"),
    "project_wrong_side": ("latent_project", "return to_f64(x) @ to_f64(a)",
                           "return (to_f64(a).T @ to_f64(x).T).T[::-1]"),
    "append_truncates": ("append_rows_bf16", "return (keep + up.astype(np.uint64)).astype(np.uint16)",
                         "return keep.astype(np.uint16)"),
    "append_ties_up": ("append_rows_bf16", "(rest == 0x8000) & ((keep & np.uint64(1)) == 1)",
                       "(rest == 0x8000)"),
    "bf16_widen_shift_8": ("to_f64", "<< np.uint32(16)", "<< np.uint32(8)"),
    "bf16_widen_as_fp16": ("to_f64",
                           "return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)",
                           "return a.view(np.float16).astype(np.float64)"),
    "bf16_widen_as_integer": ("to_f64",
                              "return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)",
                              "return a.astype(np.float64)"),
    "append_i4_uses_i8_quantiser": ("append_rows_i4", "return quantize_rows_i4(",
                                    "return quantize_rows_i8("),
    "append_i8_uses_i4_quantiser": ("append_rows_i8", "return quantize_rows_i8(",
                                    "return quantize_rows_i4("),
    "append_i8_via_bf16": ("append_rows_i8",
                           "np.asarray(h64, dtype=np.float64).astype(np.float32)",
                           "(append_rows_bf16(h64).astype(np.uint32) << np.uint32(16)).view(np.float32)"),
    "hadamard_i4_rotation_dropped": ("append_rows_i4_hadamard",
                                     "quantize_rows_i4((h @ hadamard(h.shape[-1])).astype(np.float32))",
                                     "quantize_rows_i4(h.astype(np.float32))"),
    "hadamard_i4_uses_i8": ("append_rows_i4_hadamard", "return quantize_rows_i4(",
                            "return quantize_rows_i8("),
}

PINS = [name for name in dir(P) if name.startswith("test_")]


def _mutated_module(fn_name, old, new):
    src = inspect.getsource(O)
    fn_src = inspect.getsource(getattr(O, fn_name))
    assert old in fn_src, (fn_name, old)
    src = src.replace(fn_src, fn_src.replace(old, new))
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_pins(monkeypatch, mod):
    with open(GOLDEN) as f:
        golden = json.load(f)
    monkeypatch.setattr(P, "O", mod)
    failed = []
    for name in PINS:
        fn = getattr(P, name)
        params = inspect.signature(fn).parameters
        marks = getattr(fn, "pytestmark", [])
        grids = [m for m in marks if m.name == "parametrize"]
        calls = [{}]
        for m in grids:
            argnames = [a.strip() for a in (m.args[0].split(",") if isinstance(m.args[0], str) else m.args[0])]
            new = []
            for c in calls:
                for v in m.args[1]:
                    v = v if len(argnames) > 1 else (v,)
                    new.append({**c, **dict(zip(argnames, v))})
            calls = new
        for kw in calls:
            if "golden" in params:
                kw = {**kw, "golden": golden}
            try:
                fn(**kw)
            except (AssertionError, ValueError, IndexError):
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    mod = _mutated_module(*MUTANTS[mutant])
    failed = _run_pins(monkeypatch, mod)
    assert failed, f"no pin caught mutant {mutant}"


def test_unmutated_oracle_passes_all_pins(monkeypatch):
    assert _run_pins(monkeypatch, O) == []
