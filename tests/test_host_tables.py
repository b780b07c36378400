"""The library's host-built constant tables (csrc/tables.cpp, compiled here with
the host compiler alone) against the oracle's independently built window,
filterbank and quantizer: the window, the FFT twiddles, the mel filterbank in
the segment form the kernel uses, with the weights evaluated as the kernel
evaluates them (fp32, from each segment's edges), and the quantizer edges,
for the released configuration and others."""

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
#include <cstdlib>
#include <cstring>
#include "internal.h"
int main(int argc, char** argv) {
  static dmel::HostTables t;
  const int n_mels = std::atoi(argv[1]), n_levels = std::atoi(argv[2]);
  const float lo = std::strtof(argv[3], nullptr), hi = std::strtof(argv[4], nullptr);
  if (!dmel::build_host_tables(&t, n_mels, n_levels, lo, hi)) return 2;
  for (int i = 0; i < dmel::kWindow; ++i) std::printf("w %d %.9g\n", i, t.window[i]);
  for (int i = 0; i < dmel::kHalf; ++i) std::printf("t8 %d %.9g %.9g\n", i, t.tw800[2 * i], t.tw800[2 * i + 1]);
  for (int i = 0; i <= dmel::kHalf / 2; ++i) std::printf("t16 %d %.9g %.9g\n", i, t.tw1600[2 * i], t.tw1600[2 * i + 1]);
  for (int i = 0; i < 24 * 32; ++i) std::printf("ta %d %.9g %.9g\n", i, t.twa[2 * i], t.twa[2 * i + 1]);
  for (int i = 0; i < n_mels + 2; ++i) std::printf("ss %d %d\n", i, t.seg_start[i]);
  for (int i = 0; i <= n_mels; ++i) std::printf("sg %d %.9g %.9g %.9g\n", i, t.seg_lo[i], t.seg_hi[i], t.seg_inv[i]);
  for (int i = 0; i <= n_levels; ++i) std::printf("qe %d %.9g\n", i, t.q_edge[i]);
  for (int i = 0; i < 32; ++i) std::printf("mr %d %d\n", i, t.mel_round[i]);
  for (int i = 0; i < 4 * dmel::kMelMaxSides * 8; ++i) std::printf("mf %d %d %d\n", i, t.mel_first[i], t.mel_filt[i]);
  for (int i = 0; i < dmel::kMelChunks * 64; ++i) std::printf("mw %d %.9g\n", i, t.mel_w[i]);
  for (int i = 0; i < dmel::kImgFull; ++i) {
    unsigned u;
    std::memcpy(&u, &t.lds_image[i], 4);
    std::printf("im %d %u\n", i, u);
  }
  std::printf("ml 0 %d\n", t.mel_in_lds);
  std::printf("kc 0 %d %d %d %d %d %d %d %d %d\n", dmel::kMelMaxSides, dmel::kMelChunks, dmel::kMelReadEnd,
              dmel::kImgWindow, dmel::kImgTwa, dmel::kImgTw1600, dmel::kImgEdge, dmel::kImgMelW, dmel::kMelLdsChunks);
  std::printf("kd 0 %d %d\n", dmel::kImgMelFirst, dmel::kImgMelFilt);
  return 0;
}
"""


CONFIGS = [(80, 16, -7.0, 2.0), (80, 16, -1.5, 2.0), (40, 8, -5.0, 1.0), (128, 10, -7.0, 2.0),
           (1, 1, -7.0, 2.0), (64, 256, -3.0, 4.5)]


@pytest.fixture(scope="module")
def dump_exe(tmp_path_factory):
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
    return exe


def _dump(exe, cfg):
    out = subprocess.run([str(exe)] + [repr(v) for v in cfg], check=True, capture_output=True, text=True).stdout
    t = {"w": {}, "t8": {}, "t16": {}, "ta": {}, "ss": {}, "sg": {}, "qe": {}, "mr": {}, "mf": {}, "mw": {},
         "im": {}, "ml": {}, "kc": {}, "kd": {}}
    for line in out.splitlines():
        k, i, *v = line.split()
        t[k][int(i)] = [float(x) for x in v]
    return t


@pytest.fixture(scope="module")
def tables(dump_exe):
    return _dump(dump_exe, CONFIGS[0])


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


@pytest.mark.parametrize("cfg", CONFIGS)
def test_segment_filterbank_matches_oracle(dump_exe, cfg):
    tables = _dump(dump_exe, cfg)
    n = cfg[0]
    H = o.mel_filterbank(n)
    starts = [tables["ss"][i][0] for i in range(n + 2)]
    assert starts[0] == 0 and starts[n + 1] == 801 and all(a <= b for a, b in zip(starts, starts[1:]))
    G = np.zeros((n, 801))
    tol = np.zeros((n, 801))
    bin_hz = np.float32(16000.0 / 1600.0)
    for s in range(n + 1):
        lo, hi, inv = (np.float32(v) for v in tables["sg"][s])
        for k in range(int(starts[s]), int(starts[s + 1])):
            fk = np.float32(bin_hz * np.float32(k))
            rise = np.float32(np.float32(fk - lo) * inv)
            fall = np.float32(np.float32(hi - fk) * inv)
            # fp32 rounding of f, the edges, 1/(hi - lo), the difference and
            # the product: a few ulps of (f + hi) / (hi - lo)
            bound = 4.0 * 2.0 ** -24 * (float(fk) + float(hi)) * float(inv) + 1e-12
            if s < n:
                G[s, k] += rise
                tol[s, k] = bound
            if s > 0:
                G[s - 1, k] += fall
                tol[s - 1, k] = bound
    # every bin lies between the edges of its segment, and the weights agree
    # with the oracle's fp64 triangles to fp32 rounding
    assert np.all(np.abs(G - H) <= tol)
    assert np.max(np.abs(G - H)) < 2e-5
    assert np.array_equal(G > 1e-6, H > 1e-6)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_quantizer_edges_match_oracle(dump_exe, cfg):
    n_mels, n_lv, lo, hi = cfg
    t = _dump(dump_exe, cfg)
    q = np.array([t["qe"][i][0] for i in range(n_lv + 1)], dtype=np.float32)
    assert q[0] == np.float32(lo) and q[-1] == np.float32(hi)
    e = o.level_edges(lo, hi, n_lv)
    # each stored edge is the smallest fp32 value >= the oracle's fp64 edge
    inner = q[1:-1].astype(np.float64)
    below = np.nextafter(q[1:-1], np.float32(-np.inf)).astype(np.float64)
    assert np.all(inner >= e) and np.all(below < e)
    # hence the fp32 comparison decides as the oracle does on fp32 inputs
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(lo - 1, hi + 1, 20000).astype(np.float32), q, below.astype(np.float32)])
    c = np.minimum(np.maximum(x, np.float32(lo)), np.float32(hi))
    lv = (c[:, None] >= q[None, 1:-1]).sum(axis=1)
    assert np.array_equal(lv, o.quantize(x.astype(np.float64), lo, hi, n_lv))


def _schedule(t):
    """The filter schedule as the kernel reads it: {filter: [(bin, weight)]},
    plus the reads of every (round, side, slot) as (first bin, chunks, slot)."""
    n_sides, n_chunks, read_end = (int(v) for v in t["kc"][0][:3])
    rnd = [int(t["mr"][i][0]) for i in range(32)]
    first = {i: int(v[0]) for i, v in t["mf"].items()}
    filt = {i: int(v[1]) for i, v in t["mf"].items()}
    mw = np.array([t["mw"][i][0] for i in range(n_chunks * 64)]).reshape(n_chunks, 2, 8, 4)
    taps, reads = {}, []
    for r in range(4):
        base, chunks, sides = rnd[8 * r], rnd[8 * r + 1], rnd[8 * r + 2]
        st = rnd[8 * r + 3: 8 * r + 3 + n_sides + 1]
        assert st[0] == 0 and st[sides] == chunks and all(a <= b for a, b in zip(st, st[1:sides + 1]))
        for h in range(sides):
            for slot in range(8):
                i = 8 * (n_sides * r + h) + slot
                pb, j = first[i], filt[i]
                reads.append((pb, st[h + 1] - st[h], slot))
                for c in range(st[h], st[h + 1]):
                    for q in range(8):
                        w = mw[base + c, q // 4, slot, q % 4]
                        if j < 0:
                            assert w == 0.0
                        elif w != 0.0:
                            taps.setdefault(j, []).append((pb + 8 * (c - st[h]) + q, w))
                if j >= 0:
                    taps.setdefault(j, [])
    return taps, reads, read_end


@pytest.mark.parametrize("cfg", CONFIGS)
def test_filter_schedule_matches_oracle(dump_exe, cfg):
    """Every filter once, its weights the oracle's triangle (times the kernel's
    1/4) to fp32 rounding, no weight outside its bin range, and every read of
    the kernel inside [-8, kMelReadEnd) with the 8 slots of a side starting at
    bins distinct mod 8."""
    t = _dump(dump_exe, cfg)
    n = cfg[0]
    taps, reads, read_end = _schedule(t)
    assert sorted(taps) == list(range(n))
    H = o.mel_filterbank(n)
    starts = [int(t["ss"][i][0]) for i in range(n + 2)]
    for j in range(n):
        W = np.zeros(801)
        for k, w in taps[j]:
            assert starts[j] <= k < starts[j + 2], (j, k)
            W[k] += 4.0 * w
        assert np.all(np.abs(W - H[j]) <= 2.0 ** -22 * np.abs(H[j]) + 1e-12), j
    for pb, chunks, slot in reads:
        assert pb >= -8 and pb + 8 * chunks <= read_end
        assert pb % 8 == slot


@pytest.mark.parametrize("cfg", CONFIGS)
def test_lds_image(dump_exe, cfg):
    """The table image the kernel copies into LDS holds the window's first
    half and middle, the pass-A and split twiddles, the quantizer edges and,
    when it fits, the schedule."""
    t = _dump(dump_exe, cfg)
    _, _, _, k_win, k_twa, k_t16, k_edge, k_mw, lds_chunks = (int(v) for v in t["kc"][0])
    k_first, k_filt = (int(v) for v in t["kd"][0])
    img = np.array([t["im"][i][0] for i in range(len(t["im"]))], dtype=np.uint32)
    f32 = img.view(np.float32)
    w = np.array([t["w"][i][0] for i in range(1600)], dtype=np.float32)
    assert np.array_equal(f32[k_win:k_win + 801], w[:801])
    assert np.array_equal(w[1:800], w[1599:800:-1])  # the half the kernel mirrors
    ta = np.array([t["ta"][i] for i in range(24 * 32)], dtype=np.float32).reshape(-1)
    assert np.array_equal(f32[k_twa:k_twa + ta.size], ta)
    t16 = np.array([t["t16"][i] for i in range(401)], dtype=np.float32).reshape(-1)
    assert np.array_equal(f32[k_t16:k_t16 + t16.size], t16)
    qe = np.array([t["qe"][i][0] for i in range(cfg[1] + 1)], dtype=np.float32)
    assert np.array_equal(f32[k_edge:k_edge + qe.size], qe)
    rnd = [int(t["mr"][i][0]) for i in range(32)]
    total = rnd[24] + rnd[25]
    in_lds = int(t["ml"][0][0])
    assert in_lds == (total <= lds_chunks)
    if in_lds:
        mw = np.array([t["mw"][i][0] for i in range(total * 64)], dtype=np.float32)
        assert np.array_equal(f32[k_mw:k_mw + mw.size], mw)
        mf = t["mf"]
        first = np.array([int(mf[i][0]) for i in range(len(mf))], dtype=np.int32)
        filt = np.array([int(mf[i][1]) for i in range(len(mf))], dtype=np.int32)
        assert np.array_equal(img[k_first:k_first + first.size].view(np.int32), first)
        assert np.array_equal(img[k_filt:k_filt + filt.size].view(np.int32), filt)


def test_filter_schedule_every_count(dump_exe):
    """Every filter count the configuration allows builds a schedule (the
    library would refuse the context otherwise) whose filters all appear."""
    for n in (1, 2, 3, 7, 8, 9, 31, 32, 33, 47, 63, 64, 65, 96, 100, 127, 128):
        t = _dump(dump_exe, (n, 16, -7.0, 2.0))
        taps, reads, read_end = _schedule(t)
        assert sorted(taps) == list(range(n)), n
