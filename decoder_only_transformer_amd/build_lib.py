"""Builds libllama_mi355x.so in-tree with hipcc for gfx950.

    python -m decoder_only_transformer_amd.build_lib

Each HIP source is compiled to an object in parallel, then linked into one shared library
next to this file.  All device code is built with the packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libllama_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["gemv.hip", "gemm.hip", "attention.hip", "flash_attention.hip", "skinny.hip", "misc.hip", "sampling.hip",
           "llama_api.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the host library code (the C ABI's
# validation and launch plan); device code is never built with them.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SAN_LIB = os.path.join(HERE, "_build", "libllama_mi355x_san.so")


def _compile(src: str, obj: str, extra=()) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every source and link the library; returns its path.  sanitize=True builds the
    host-sanitized variant (the host code of llama_api.cpp with SAN_HOST) as SAN_LIB instead."""
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="llama_build_") as tmp:
        objs = [os.path.join(tmp, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
        extras = [SAN_HOST if (sanitize and s == "llama_api.cpp") else () for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
            list(ex.map(_compile, SOURCES, objs, extras))
        tmp_lib = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_lib, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
