"""Build libmxfp4.so in-tree with hipcc for gfx950.

    python -m mxfp4_microscaled_precision_amd.build

Every source is compiled on each call (a rebuild is cheap and the library
must always match its sources).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libmxfp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["mx_quant.hip", "mx_gemm.hip", "mx_gemm_e4m3.hip", "mx_dequant.hip", "mx_api.cpp"]

# -ffp-contract=off: the rotation's adds and multiplies must round one by one.
# -packed-fp32-ops off: packed fp32 VALU forms are not used by this library.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-gpu-rdc",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found: cannot build the gfx950 library")
    return cand


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libmxfp4.so next to this file."""
    objs = []
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    flags = list(HIP_FLAGS) + list(extra_flags or [])
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [hipcc()] + flags + lang + ["-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
