"""Builds libdmel.so (gfx950) in place with hipcc, and libdmel_bench.so, the
benchmark-only companion library (csrc/bench) that links against it.

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
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libdmel_bench.so")

SOURCES = ["dmel_api.cpp", "tables.cpp", "frontend.hip", "embed.hip", "shortconv.hip", "backward.hip", "hmlp.hip",
           "noalloc.hip"]
BENCH_SOURCES = ["bench/bench_api.cpp", "bench/dft_gemm.hip", "bench/rounding_probe.hip", "bench/valu_rate.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are switched off (they are never needed for
# correctness here, and the plain-VALU sum is the one whose rounding is pinned).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, build_dir: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(build_dir, os.path.splitext(src.replace("/", "_"))[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           "-I", INCLUDE, "-I", CSRC, "-I", os.path.join(CSRC, "bench"), "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_FLAGS
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    _run(cmd, verbose)
    return obj


def _link(objs, out: str, extra, verbose: bool) -> None:
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + extra, verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compiles every source for gfx950 and links libdmel.so and
    libdmel_bench.so next to this file."""
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    _link([_compile(s, build_dir, verbose) for s in SOURCES], LIB_PATH, [], verbose)
    _link([_compile(s, build_dir, verbose) for s in BENCH_SOURCES], BENCH_LIB_PATH,
          ["-L" + PKG_DIR, "-ldmel", "-Wl,-rpath,$ORIGIN"], verbose)
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
