"""Pins for the short-convolution oracle: a hand-worked example, the
per-channel full convolution of numpy (a textbook routine), the impulse
response (which fixes the direction of the taps), chunked streaming with the
state equal to one pass, causality and linearity."""

import json
import os

import numpy as np

from oracle import shortconv_oracle as sc


def _bits(v):
    a = np.asarray(v, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_values(rng, shape, scale=1.0):
    # values exact in bf16: rounded through the bit pattern
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return sc.bf16_bits_to_f64(_bits(v))


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "shortconv_worked.json")) as f:
        g = json.load(f)
    y, st = sc.shortconv(_bits(g["x"]), g["seq_off"], np.array(g["weight"]), _bits(g["state_in"]))
    assert np.array_equal(y, np.array(g["y"]))
    assert np.array_equal(sc.bf16_bits_to_f64(st), np.array(g["state_out"]))


def test_matches_numpy_convolve():
    rng = np.random.default_rng(1)
    C, lens = 5, [0, 1, 2, 3, 17]
    x = _bf16_values(rng, (sum(lens), C))
    st = _bf16_values(rng, (len(lens), 3, C))
    w = rng.uniform(-1, 1, (C, 4))
    off = np.concatenate([[0], np.cumsum(lens)])
    y, _ = sc.shortconv(_bits(x), off, w, _bits(st))
    for s, n in enumerate(lens):
        a = off[s]
        for c in range(C):
            xp = np.concatenate([st[s, :, c], x[a:a + n, c]])
            full = np.convolve(xp, w[c])          # full[k] = sum_d w[d] xp[k - d]
            want = x[a:a + n, c] + full[3:3 + n]
            assert np.allclose(y[a:a + n, c], want, rtol=0, atol=1e-12)


def test_impulse_response_fixes_tap_direction():
    C, T = 3, 10
    w = np.array([[0.5, 0.25, 0.125, 0.0625], [1.0, 2.0, 3.0, 4.0], [-1.0, 0.0, 0.0, 1.0]])
    x = np.zeros((T, C))
    x[4, :] = 1.0
    y, _ = sc.shortconv(_bits(x), [0, T], w)
    for c in range(C):
        want = np.zeros(T)
        want[4] = 1.0 + w[c, 0]
        want[5:8] = w[c, 1:4]
        assert np.array_equal(y[:, c], want)


def test_chunked_with_state_equals_one_pass():
    rng = np.random.default_rng(2)
    C, n = 7, 50
    x = _bf16_values(rng, (n, C))
    w = rng.uniform(-1, 1, (C, 4))
    y_all, st_all = sc.shortconv(_bits(x), [0, n], w)
    cuts = [0, 1, 1, 3, 4, 20, 22, 50]
    state = None
    ys = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        y, state = sc.shortconv(_bits(x[a:b]), [0, b - a], w, state)
        ys.append(y)
    assert np.array_equal(np.concatenate(ys), y_all)
    assert np.array_equal(state, st_all)


def test_causal_and_linear():
    rng = np.random.default_rng(3)
    C, n = 4, 30
    x = _bf16_values(rng, (n, C))
    w = rng.uniform(-1, 1, (C, 4))
    y, _ = sc.shortconv(_bits(x), [0, n], w)
    x2 = x.copy()
    x2[20:] = _bf16_values(rng, (n - 20, C))
    y2, _ = sc.shortconv(_bits(x2), [0, n], w)
    assert np.array_equal(y[:20], y2[:20])
    # zero weights: the residual alone
    y0, _ = sc.shortconv(_bits(x), [0, n], np.zeros((C, 4)))
    assert np.array_equal(y0, x)
    # doubling the input doubles the output (exact: powers of two)
    yd, _ = sc.shortconv(_bits(2 * x), [0, n], w)
    assert np.array_equal(yd, 2 * y)
