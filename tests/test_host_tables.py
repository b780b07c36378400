"""The library's host-built constant tables (csrc/tables.cpp, compiled here with
the host compiler alone) against the oracle's independently built window and
filterbank: the window, the FFT twiddles and the mel filterbank in the
segment form the kernel uses, with the weights evaluated as the kernel
evaluates them (fp32, from each segment's edges)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import dmel_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "encoder_free_audio_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "internal.h"
int main() {
  static dmel::HostTables t;
  dmel::build_host_tables(&t);
  for (int i = 0; i < dmel::kWindow; ++i) std::printf("w %d %.9g\n", i, t.window[i]);
  for (int i = 0; i < dmel::kHalf; ++i) std::printf("t8 %d %.9g %.9g\n", i, t.tw800[2 * i], t.tw800[2 * i + 1]);
  for (int i = 0; i <= dmel::kHalf / 2; ++i) std::printf("t16 %d %.9g %.9g\n", i, t.tw1600[2 * i], t.tw1600[2 * i + 1]);
  for (int i = 0; i < 24 * 32; ++i) std::printf("ta %d %.9g %.9g\n", i, t.twa[2 * i], t.twa[2 * i + 1]);
  for (int i = 0; i < dmel::kMels + 2; ++i) std::printf("ss %d %d\n", i, t.seg_start[i]);
  for (int i = 0; i <= dmel::kMels; ++i) std::printf("sg %d %.9g %.9g %.9g\n", i, t.seg_lo[i], t.seg_hi[i], t.seg_inv[i]);
  return 0;
}
"""


@pytest.fixture(scope="module")
def tables(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("tables")
    src = d / "dump.cpp"
    src.write_text(DRIVER)
    exe = d / "dump"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run([gxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                    "-I", CSRC, "-I", os.path.join(ROOT, "include"), str(src), os.path.join(CSRC, "tables.cpp"),
                    "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    t = {"w": {}, "t8": {}, "t16": {}, "ta": {}, "ss": {}, "sg": {}}
    for line in out.splitlines():
        k, i, *v = line.split()
        t[k][int(i)] = [float(x) for x in v]
    return t


def test_window(tables):
    w = np.array([tables["w"][i][0] for i in range(1600)])
    assert np.max(np.abs(w - o.hann_window())) < 1e-7


def test_twiddles(tables):
    t8 = np.array([tables["t8"][i] for i in range(800)])
    m = np.arange(800)
    assert np.max(np.abs(t8[:, 0] + 1j * t8[:, 1] - np.exp(-2j * np.pi * m / 800))) < 1e-7
    t16 = np.array([tables["t16"][i] for i in range(401)])
    k = np.arange(401)
    assert np.max(np.abs(t16[:, 0] + 1j * t16[:, 1] - np.exp(-2j * np.pi * k / 1600))) < 1e-7
    ta = np.array([tables["ta"][i] for i in range(24 * 32)]).reshape(24, 32, 2)
    k2 = np.arange(1, 25)[:, None]
    n1 = np.arange(32)[None, :]
    want = np.exp(-2j * np.pi * n1 * k2 / 800)
    assert np.max(np.abs(ta[..., 0] + 1j * ta[..., 1] - want)) < 1e-7


def test_segment_filterbank_matches_oracle(tables):
    H = o.mel_filterbank()
    starts = [tables["ss"][i][0] for i in range(82)]
    assert starts[0] == 0 and starts[81] == 801 and all(a <= b for a, b in zip(starts, starts[1:]))
    G = np.zeros((80, 801))
    bin_hz = np.float32(16000.0 / 1600.0)
    for s in range(81):
        lo, hi, inv = (np.float32(v) for v in tables["sg"][s])
        for k in range(int(starts[s]), int(starts[s + 1])):
            fk = np.float32(bin_hz * np.float32(k))
            rise = np.float32(np.float32(fk - lo) * inv)
            fall = np.float32(np.float32(hi - fk) * inv)
            if s < 80:
                G[s, k] += rise
            if s > 0:
                G[s - 1, k] += fall
    # every bin lies between the edges of its segment, and the weights agree
    # with the oracle's fp64 triangles to fp32 rounding
    assert np.max(np.abs(G - H)) < 2e-6
    assert np.array_equal(G > 1e-6, H > 1e-6)
