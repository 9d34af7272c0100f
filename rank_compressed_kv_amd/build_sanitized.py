"""Build libpalu_san.so: the library with its host layer (api.cpp) compiled
with AddressSanitizer and UndefinedBehaviorSanitizer, for the ABI tests on the
CPU. Not used on a GPU.

    python -m rank_compressed_kv_amd.build_sanitized
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from rank_compressed_kv_amd.build import (ARCH, BUILD, COMMON, CSRC, INCLUDE, _compile, hipcc,
                                          sources)

# Host sanitizers for the C ABI layer (api.cpp: validation, planning,
# workspace arithmetic): address and undefined-behaviour checks on the host
# pass only (each flag behind -Xarch_host, so no GPU code is built with
# them). The kernels' objects are those of the ordinary build.
SANITIZE = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
            "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_LIB = os.path.join(BUILD, "libpalu_san.so")


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (to preload into an uninstrumented
    Python that loads the sanitized library)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    if not path:
        raise RuntimeError("the ASan runtime of the ROCm compiler was not found")
    return path


def build(verbose: bool = False) -> str:
    """libpalu_san.so: api.cpp built with host ASan + UBSan, linked with the
    kernel objects (rebuilt when a source or header is newer than them)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    newest = max(os.path.getmtime(f) for f in
                 srcs + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
                 + [os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE)])
    kernels = [f for f in srcs if not f.endswith("api.cpp")]
    objs = []
    stale = []
    for src in kernels:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < newest:
            stale.append(src)
        objs.append(obj)
    if stale:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(stale))) as ex:
            list(ex.map(_compile, stale))
    api = [f for f in srcs if f.endswith("api.cpp")][0]
    san_obj = os.path.join(BUILD, "api_san.o")
    flags = [c for c in COMMON if c != "-O3"]
    cmd = [hipcc(), *flags, *SANITIZE, "-c", api, "-o", san_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           san_obj, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
