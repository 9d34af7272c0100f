"""Summaries of rocprofv3 output for the benchmark's roofline (not used by the
library itself).

    python -m rank_compressed_kv_amd.profiling stats <run_kernel_stats.csv>
        kernel time table (markdown) of a --kernel-trace --stats run
    python -m rank_compressed_kv_amd.profiling counters <dir> [<dir> ...]
        per-kernel means of every counter in the run_counter_collection.csv of
        each --pmc pass directory, with derived per-wave figures (markdown)
    python -m rank_compressed_kv_amd.profiling traffic [label:]<fetch_dir>,<write_dir> ...
        HBM bytes per launch from a FETCH_SIZE pass and a WRITE_SIZE pass of a
        run that copies 1 GiB on the device first (bench.py --copy-probe or
        --profile-calls), scaled by what the counters read for that copy;
        each pair's kernels are recorded under their names, with " | label"
        when a label is given (a variant such as "hadamard"); writes
        profiles/traffic.json (which bench.py reads) and prints the markdown
        table

A traffic record is tied to the source files of its kernel: bench.py reports
it only while their SHA-256 is unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import OrderedDict, defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_BYTES = 1 << 30            # the bench's --copy-probe copy
# the sources whose code decides each traced kernel's memory traffic
KERNEL_SOURCES = {
    "split_absorbed_mfma_kernel": ["decode_absorbed_mfma.hip", "device_util.h"],
    "split_absorbed_int_kernel": ["decode_absorbed_quant.hip", "device_util.h"],
    "merge_fast_kernel": ["absorb_merge.hip", "device_util.h"],
    "absorb_q_vec_kernel": ["absorb_merge.hip", "absorb_device.h", "device_util.h"],
    "append_kernel": ["latent_append.hip", "absorb_device.h", "device_util.h"],
    "append_t_kernel": ["latent_append_t.hip", "absorb_device.h", "device_util.h"],
    "split_reconstruct_wave_kernel": ["decode_reconstruct_wave.hip", "reconstruct_wave_util.h",
                                      "device_util.h"],
    "split_reconstruct_wide_kernel": ["decode_reconstruct_wide.hip", "reconstruct_wave_util.h",
                                      "device_util.h"],
    "split_reconstruct_quarter_kernel": ["decode_reconstruct_quarter.hip", "reconstruct_wave_util.h",
                                      "device_util.h"],
    "split_reconstruct_mfma_kernel": ["decode_reconstruct_mfma.hip", "device_util.h"],
}


def short_name(name: str) -> str:
    """'void palu::(anonymous namespace)::k<256, false>(palu::DecodeParams)' ->
    'k<256, false>'."""
    n = name
    if n.startswith("void "):
        n = n[5:]
    if "(" in n:
        depth, cut = 0, len(n)
        for i, ch in enumerate(n):           # the argument list after the template
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
            elif ch == "(" and depth == 0 and i > 0 and n[i - 1] != ":":
                cut = i
        n = n[:cut]
    return n.split("::")[-1] if "::" in n.split("<")[0] else n


def base_name(name: str) -> str:
    return short_name(name).split("<")[0]


def sources_sha(kernel: str):
    files = KERNEL_SOURCES.get(base_name(kernel))
    if not files:
        return None, None
    h = hashlib.sha256()
    rels = [os.path.join("rank_compressed_kv_amd", "csrc", f) for f in files]
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return rels, h.hexdigest()


def read_counters(path: str):
    """{kernel: {counter: [value per dispatch]}} of one counter collection."""
    out = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def _collection(d: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"{d}: expected one counter_collection.csv, found {len(hits)}")
    return hits[0]


def cmd_stats(path: str) -> None:
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")


def cmd_counters(dirs) -> None:
    merged = defaultdict(dict)
    for d in dirs:
        for k, cs in read_counters(_collection(d)).items():
            for c, v in cs.items():
                merged[k][c] = sum(v) / len(v)
    for k, cs in merged.items():
        if k.startswith("__amd") or "at::native" in k:
            continue
        print(f"### `{short_name(k)}`\n")
        print("| counter | mean per dispatch |")
        print("|---|---:|")
        for c in sorted(cs):
            print(f"| {c} | {cs[c]:.6g} |")
        waves = cs.get("SQ_WAVES")
        if waves:
            print()
            derived = OrderedDict()
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                      "SQ_INSTS_VMEM"):
                if c in cs:
                    derived[f"{c} per wave"] = cs[c] / waves
            if "SQ_INSTS_VALU" in cs and "SQ_INSTS_MFMA" in cs:
                derived["non-MFMA VALU per wave"] = (cs["SQ_INSTS_VALU"] - cs["SQ_INSTS_MFMA"]) / waves
            if "SQ_WAVE_CYCLES" in cs:
                for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                          "SQ_ACTIVE_INST_ANY"):
                    if c in cs:
                        derived[f"{c} / SQ_WAVE_CYCLES"] = cs[c] / cs["SQ_WAVE_CYCLES"]
            if "SQ_LDS_BANK_CONFLICT" in cs and "SQ_ACTIVE_INST_LDS" in cs:
                derived["SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS"] = (
                    cs["SQ_LDS_BANK_CONFLICT"] / cs["SQ_ACTIVE_INST_LDS"])
            if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and "GRBM_GUI_ACTIVE" in cs:
                # MFMA busy cycles summed over the SIMDs (1024), GUI_ACTIVE over
                # the eight XCDs: the matrix cores' busy fraction
                derived["MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / "
                        "(GRBM_GUI_ACTIVE / 8 XCDs))"] = (
                    cs["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (cs["GRBM_GUI_ACTIVE"] / 8))
            print("| derived | value |")
            print("|---|---:|")
            for c, v in derived.items():
                print(f"| {c} | {v:.4g} |")
        print()


def cmd_traffic(pairs) -> None:
    rec = {"calibration": {}, "kernels": {}}
    print("| kernel | variant | launches | FETCH_SIZE KB | WRITE_SIZE KB | fetch / write "
          "scale | HBM read MB | HBM write MB |")
    print("|---|---|---:|---:|---:|---:|---:|---:|")
    for pair in pairs:
        label, dirs = pair.split(":", 1) if ":" in pair else ("", pair)
        fetch_dir, write_dir = dirs.split(",")
        fetch = read_counters(_collection(fetch_dir))
        write = read_counters(_collection(write_dir))

        def copy_value(data, counter):
            vals = [v for k, cs in data.items() if k.startswith("__amd_rocclr_copyBuffer")
                    for v in cs.get(counter, [])]
            return max(vals) if vals else None

        f_copy, w_copy = copy_value(fetch, "FETCH_SIZE"), copy_value(write, "WRITE_SIZE")
        if not f_copy or not w_copy:
            raise SystemExit(f"{pair}: no 1 GiB copy in the passes")
        f_scale = COPY_BYTES / (f_copy * 1024)
        w_scale = COPY_BYTES / (w_copy * 1024)
        rec["calibration"][label or "plain"] = {"fetch": f_scale, "write": w_scale,
                                                "copy_fetch_kb": f_copy, "copy_write_kb": w_copy}
        for k in fetch:
            if k.startswith("__amd") or "at::native" in k or k not in write:
                continue
            fv, wv = fetch[k]["FETCH_SIZE"], write[k]["WRITE_SIZE"]
            fkb, wkb = sum(fv) / len(fv), sum(wv) / len(wv)
            rd, wr = fkb * 1024 * f_scale, wkb * 1024 * w_scale
            rels, sha = sources_sha(k)
            name = short_name(k)
            key = f"{name} | {label}" if label else name
            rec["kernels"][key] = {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr,
                                   "sources": rels, "sources_sha256": sha}
            print(f"| `{name}` | {label or '-'} | {len(fv)} | {fkb:.1f} | {wkb:.1f} | "
                  f"{f_scale:.4f} / {w_scale:.4f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} |")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)


def main(argv) -> None:
    if len(argv) >= 2 and argv[0] == "stats":
        cmd_stats(argv[1])
    elif len(argv) >= 2 and argv[0] == "counters":
        cmd_counters(argv[1:])
    elif len(argv) >= 2 and argv[0] == "traffic":
        cmd_traffic(argv[1:])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
