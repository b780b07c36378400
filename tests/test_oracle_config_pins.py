"""Pins for the oracle's configurable front end: the parametric quantizer
(clamp range and level count from the config keys dmel_min_value,
dmel_max_value and mel_vocab_size), other mel-bin counts (n_mel_bins) and the
table layout with another number of rows per bin.

The checks compare with hand-worked values for the serving default clamp
minimum -1.5, with the floor formula evaluated in exact rational arithmetic,
with closed forms of the HTK filterbank, and with integer sums.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dmel_oracle as o


def test_serving_default_quantizer_golden(golden_dir):
    with open(os.path.join(golden_dir, "quantizer_serving.json")) as f:
        g = json.load(f)
    c = g["config"]
    e = o.level_edges(c["min_value"], c["max_value"], c["n_levels"])
    assert np.array_equal(e, np.array(g["edges"]))
    x = np.array([v for v, _ in g["cases"]])
    want = np.array([lv for _, lv in g["cases"]], dtype=np.uint8)
    assert np.array_equal(o.quantize(x, c["min_value"], c["max_value"], c["n_levels"]), want)
    # the fp32 neighbours of every edge fall on either side of it
    for k, edge in enumerate(g["edges"], start=1):
        below = np.nextafter(np.float32(edge), np.float32(-np.inf))
        got = o.quantize(np.array([below, np.float32(edge)], dtype=np.float32), -1.5, 2.0, 16)
        assert list(got) == [k - 1, k]


def _exact_level(x: float, lo: float, hi: float, n: int) -> int:
    c = min(max(Fraction(x), Fraction(lo)), Fraction(hi))
    y = (c - Fraction(lo)) * n / (Fraction(hi) - Fraction(lo))
    return min(n - 1, int(y.__floor__()))


@pytest.mark.parametrize("lo,hi,n", [(-7.0, 2.0, 16), (-1.5, 2.0, 16), (-7.0, 2.0, 10), (-5.0, 1.0, 8),
                                     (-3.0, 4.5, 256), (-2.0, 2.0, 3), (-7.0, 2.0, 1), (0.25, 0.5, 5)])
def test_quantizer_against_exact_floor(lo, hi, n):
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.uniform(lo - 2, hi + 2, 3000), [lo, hi, lo - 1, hi + 1]])
    x = x.astype(np.float32).astype(np.float64)
    got = o.quantize(x, lo, hi, n)
    edges = [Fraction(lo) + (Fraction(hi) - Fraction(lo)) * k / n for k in range(1, n)]
    checked = 0
    for v, g in zip(x, got):
        # skip values within 1e-12 of an exact edge (there the fp64 edge decides)
        if any(abs(Fraction(v) - e) < Fraction(1, 10 ** 12) for e in edges):
            continue
        assert g == _exact_level(v, lo, hi, n), (v, g)
        checked += 1
    assert checked > 2900
    assert got.max() <= n - 1
    assert o.quantize(np.array([lo]), lo, hi, n)[0] == 0
    assert o.quantize(np.array([hi]), lo, hi, n)[0] == n - 1


def test_quantizer_levels_evenly_spaced():
    # each level's preimage is an interval of width (hi - lo) / n inside the range
    lo, hi, n = -7.0, 2.0, 10
    grid = np.linspace(lo, hi, 900_001)
    lv = o.quantize(grid, lo, hi, n)
    assert np.all(np.diff(lv.astype(int)) >= 0)
    counts = np.bincount(lv, minlength=n)
    assert counts.max() - counts.min() <= 2
    assert o.quantize(np.array([-6.1 + 1e-9, -6.1 - 1e-9]), lo, hi, n).tolist() == [1, 0]


def test_quantizer_rejects_bad_config():
    with pytest.raises(ValueError):
        o.level_edges(2.0, -7.0, 16)
    with pytest.raises(ValueError):
        o.level_edges(-7.0, 2.0, 0)
    with pytest.raises(ValueError):
        o.quantize(np.zeros(3), -7.0, 2.0, 257)


@pytest.mark.parametrize("n_mels", [1, 2, 40, 64, 80, 128])
def test_filterbank_other_bin_counts(n_mels):
    H = o.mel_filterbank(n_mels)
    assert H.shape == (n_mels, 801)
    e = o.mel_edges_hz(n_mels)
    assert e[0] == 0.0 and e[-1] == 8000.0 and e.size == n_mels + 2
    # centre of filter j: equally spaced in HTK mel, closed form
    top = 2595.0 * np.log10(1.0 + 8000.0 / 700.0)
    j = np.arange(n_mels)
    centre = 700.0 * (10.0 ** ((j + 1) * top / (n_mels + 1) / 2595.0) - 1.0)
    assert np.allclose(e[1:-1], centre, rtol=1e-12, atol=1e-9)
    # unit peak at the centre, zero outside the outer edges
    for jj in (0, n_mels // 2, n_mels - 1):
        assert abs(o.triangle(jj, centre[jj], n_mels) - 1.0) < 1e-12
        assert o.triangle(jj, e[jj], n_mels) == 0.0 and o.triangle(jj, e[jj + 2], n_mels) == 0.0
    # partition of unity between the first and the last centre
    f = np.arange(801) * 10.0
    inner = (f >= centre[0]) & (f <= centre[-1])
    if inner.any():
        assert np.max(np.abs(H[:, inner].sum(axis=0) - 1.0)) < 1e-12
    # a bin feeds at most two filters
    assert np.max((H > 0).sum(axis=0)) <= 2


def test_filterbank_single_filter_closed_form():
    top = 2595.0 * np.log10(1.0 + 8000.0 / 700.0)
    c = 700.0 * (10.0 ** (top / 2.0 / 2595.0) - 1.0)
    f = np.arange(801) * 10.0
    want = np.minimum(f / c, (8000.0 - f) / (8000.0 - c))
    assert np.max(np.abs(o.mel_filterbank(1)[0] - want)) < 1e-12


def test_filterbank_default_unchanged():
    assert np.array_equal(o.mel_filterbank(80), o.mel_filterbank())


def test_embedding_other_layout_integer_table():
    # 40 bins x 8 levels: row = 8 * bin + level, exact integer sums
    rng = np.random.default_rng(5)
    n_bins, n_lv, d = 40, 8, 32
    vals = rng.integers(-64, 64, size=(n_bins * n_lv, d)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(o.bf16_to_f32(bits), vals)
    lv = rng.integers(0, n_lv, size=(50, n_bins)).astype(np.uint8)
    got = o.embed_sum(lv, bits, n_levels=n_lv)
    for t in range(50):
        want = [0] * d
        for b in range(n_bins):
            r = 8 * b + int(lv[t, b])
            for c in range(d):
                want[c] += int(vals[r, c])
        assert got[t].tolist() == [float(v) for v in want]
    with pytest.raises(ValueError):
        o.embed_sum(np.full((1, n_bins), n_lv, np.uint8), bits, n_levels=n_lv)


def test_levels_cfg_released_equals_default():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 0.1, 8000)
    lm, lv = o.levels_cfg(x, o.Config())
    assert np.array_equal(lv, o.levels(x)) and np.array_equal(lm, o.log_mel(x))
    lm2, lv2 = o.levels_cfg(x, o.Config(40, 8, -5.0, 1.0))
    assert lm2.shape == (10, 40) and lv2.max() <= 7
