"""Pins for the hMLP oracle: GELU values from the normal CDF, the patch count,
a brute-force evaluation of the four stages by pixel coordinates, one-hot
weights that trace pixels through the merge order, and patch locality."""

import math

import numpy as np
import pytest

from oracle import hmlp_oracle as h


def _bits(a):
    return (np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def test_gelu_values():
    # GELU(x) = x * Phi(x); Phi(1) = 0.8413447460685429 (normal table)
    g = h.gelu(np.array([0.0, 1.0, -1.0, 10.0, -10.0, 0.5]))
    assert g[0] == 0.0
    assert abs(g[1] - 0.8413447460685429) < 1e-15
    assert abs(g[2] + 0.15865525393145707) < 1e-15
    assert abs(g[3] - 10.0) < 1e-15 and abs(g[4]) < 1e-15
    assert abs(g[5] - 0.5 * 0.5 * (1 + math.erf(0.5 / math.sqrt(2)))) < 1e-16
    x = np.linspace(-4, 4, 33)
    assert np.allclose(h.gelu(x) - h.gelu(-x), x, rtol=0, atol=1e-15)


def test_patch_count():
    assert h.num_patches(1, 1280, 960) == 32 * 24
    assert h.num_patches(3, 40, 80) == 6
    with pytest.raises(ValueError):
        h.num_patches(1, 50, 40)


def _random_weights(rng, widths, scale=0.3):
    ws = []
    k_in = 75
    for k, n_out in enumerate(widths):
        w = _bits(rng.standard_normal((n_out, k_in)) * scale / np.sqrt(k_in))
        b = (rng.standard_normal(n_out) * 0.1).astype(np.float32)
        ws.append((w, b))
        k_in = 4 * n_out
    return ws


def test_brute_force_one_patch():
    # stage outputs by explicit pixel coordinates, against the reshape form
    rng = np.random.default_rng(0)
    widths = [3, 2, 2, 5]
    ws = _random_weights(rng, widths)
    img = _bits(rng.standard_normal((1, 40, 40, 3)))
    x = h.bf16_bits_to_f64(img)[0]
    W = [h.bf16_bits_to_f64(w) for w, _ in ws]
    B = [b.astype(np.float64) for _, b in ws]
    h1 = np.zeros((8, 8, widths[0]))
    for y in range(8):
        for xx in range(8):
            for o in range(widths[0]):
                s = B[0][o]
                for dy in range(5):
                    for dx in range(5):
                        for c in range(3):
                            s += W[0][o, (dy * 5 + dx) * 3 + c] * x[5 * y + dy, 5 * xx + dx, c]
                h1[y, xx, o] = s
    h1 = h.f64_to_bf16_value(h.gelu(h1))
    prev = h1
    for k in (1, 2, 3):
        side = prev.shape[0] // 2
        cur = np.zeros((side, side, widths[k]))
        for y in range(side):
            for xx in range(side):
                for o in range(widths[k]):
                    s = B[k][o]
                    for dy in range(2):
                        for dx in range(2):
                            for c in range(widths[k - 1]):
                                s += W[k][o, (dy * 2 + dx) * widths[k - 1] + c] * prev[2 * y + dy, 2 * xx + dx, c]
                    cur[y, xx, o] = s
        prev = cur if k == 3 else h.f64_to_bf16_value(h.gelu(cur))
    got = h.hmlp(img, ws)
    assert got.shape == (1, widths[3])
    assert np.allclose(got[0], prev[0, 0], rtol=1e-12, atol=1e-12)


def test_one_hot_weights_trace_the_merge_order():
    # linear stages with one-hot weights: the output must be the pixel the
    # chain of selections points at
    img = np.arange(40 * 40 * 3, dtype=np.float32).reshape(1, 40, 40, 3) / 8.0   # exact in bf16 up to 4800/8
    bits = _bits(img)
    vals = h.bf16_bits_to_f64(bits)[0]
    for (dy1, dx1, c), (q2, q3, q4) in [((0, 0, 0), (0, 0, 0)), ((4, 3, 2), (1, 2, 3)), ((2, 1, 1), (3, 0, 2))]:
        w1 = np.zeros((1, 75)); w1[0, (dy1 * 5 + dx1) * 3 + c] = 1
        w2 = np.zeros((1, 4)); w2[0, q2] = 1
        w3 = np.zeros((1, 4)); w3[0, q3] = 1
        w4 = np.zeros((1, 4)); w4[0, q4] = 1
        ws = [(_bits(w), np.zeros(1, np.float32)) for w in (w1, w2, w3, w4)]
        got = h.hmlp(bits, ws, linear=True)[0, 0]
        # child q = dy * 2 + dx at each merge, from the top
        y8 = 4 * (q4 // 2) + 2 * (q3 // 2) + (q2 // 2)
        x8 = 4 * (q4 % 2) + 2 * (q3 % 2) + (q2 % 2)
        assert got == vals[5 * y8 + dy1, 5 * x8 + dx1, c]


def test_patches_are_independent_and_row_major():
    rng = np.random.default_rng(1)
    ws = _random_weights(rng, [4, 4, 4, 6])
    img = _bits(rng.standard_normal((2, 80, 120, 3)))
    base = h.hmlp(img, ws)
    assert base.shape == (2 * 2 * 3, 6)
    img2 = img.copy()
    img2[1, 40:80, 40:80, :] = _bits(rng.standard_normal((40, 40, 3)))   # image 1, patch (1, 1)
    changed = np.any(h.hmlp(img2, ws) != base, axis=1)
    assert changed.tolist() == [False] * 6 + [False, False, False, False, True, False]
