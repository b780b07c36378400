"""Builds libdmel.so (gfx950) in place with hipcc.

Usage: ``python -m encoder_free_audio_amd.build`` (or ``build()`` from Python).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdmel.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["dmel_api.cpp", "tables.cpp", "frontend.hip", "embed.hip", "shortconv.hip", "backward.hip", "hmlp.hip", "dft_gemm.hip", "noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are switched off (they are never needed for
# correctness here, and the plain-VALU sum is the one whose rounding is pinned).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compiles every source for gfx950 and links libdmel.so next to this file."""
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            cmd += DEVICE_FLAGS
        else:
            cmd += ["-D__HIP_PLATFORM_AMD__"]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
