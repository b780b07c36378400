"""Pins for the oracle's backward: finite differences of the RMSNorm, its
closed forms, exact integer sums and the adjoint identity for the
embedding-bag gradient, and hand-worked cases of the summation order (token
order from +0; the existing gradient added to the finished sum)."""

import json
import os

import numpy as np
import pytest

from oracle import dmel_oracle as o


def _forward(s, w, eps):
    s = np.asarray(s, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(s * s, axis=1) + eps)
    return s * w[None, :] * r[:, None]


def test_rms_backward_matches_finite_differences():
    rng = np.random.default_rng(0)
    n, d, eps = 3, 24, 1e-3
    s = rng.standard_normal((n, d))
    w = rng.uniform(0.5, 1.5, d)
    dy = rng.standard_normal((n, d))
    ds, dw, _ = o.rms_backward_from_sum(s, w, dy, eps)
    h = 1e-6
    for t in range(n):
        for c in range(d):
            sp, sm = s.copy(), s.copy()
            sp[t, c] += h
            sm[t, c] -= h
            num = (np.sum(dy * _forward(sp, w, eps)) - np.sum(dy * _forward(sm, w, eps))) / (2 * h)
            assert abs(num - ds[t, c]) < 1e-7 * max(1.0, abs(num))
    for c in range(d):
        wp, wm = w.copy(), w.copy()
        wp[c] += h
        wm[c] -= h
        num = (np.sum(dy * _forward(s, wp, eps)) - np.sum(dy * _forward(s, wm, eps))) / (2 * h)
        assert abs(num - dw[c]) < 1e-7 * max(1.0, abs(num))


def test_rms_backward_closed_forms():
    rng = np.random.default_rng(1)
    d = 64
    s = rng.standard_normal((2, d))
    w = np.ones(d)
    # eps = 0: the output is invariant to scaling s, so the gradient along s is 0
    ds, _, _ = o.rms_backward_from_sum(s, w, s, eps=0.0)
    assert np.max(np.abs(ds)) < 1e-12
    # dy orthogonal to s (w = 1): ds = r dy
    dy = rng.standard_normal((2, d))
    dy -= (np.sum(dy * s, axis=1) / np.sum(s * s, axis=1))[:, None] * s
    ds, _, r = o.rms_backward_from_sum(s, w, dy, eps=1e-6)
    assert np.allclose(ds, r[:, None] * dy, rtol=1e-12, atol=1e-14)


def test_rms_backward_uses_the_forward_sum():
    rng = np.random.default_rng(2)
    lv = rng.integers(0, 16, (5, 80)).astype(np.uint8)
    tb = o.f32_to_bf16(rng.standard_normal((1280, 32)).astype(np.float32) * 0.02)
    w = rng.uniform(0.5, 1.5, 32)
    dy = rng.standard_normal((5, 32))
    ds, dw, s, r = o.rms_backward(lv, tb, w, dy)
    assert np.array_equal(s, o.embed_sum(lv, tb))
    ds2, dw2, r2 = o.rms_backward_from_sum(s, w, dy)
    assert np.array_equal(ds, ds2) and np.array_equal(dw, dw2)


@pytest.mark.parametrize("n_bins,n_levels", [(80, 16), (40, 8), (3, 5)])
def test_embed_backward_integer_sums(n_bins, n_levels):
    rng = np.random.default_rng(3 + n_bins)
    n, d = 300, 8
    lv = rng.integers(0, n_levels, (n, n_bins)).astype(np.uint8)
    g = rng.integers(-50, 50, (n, d)).astype(np.float32)
    got = o.embed_backward(lv, g, n_levels)
    want = np.zeros((n_bins * n_levels, d), dtype=np.int64)
    for t in range(n):
        for b in range(n_bins):
            want[n_levels * b + int(lv[t, b])] += g[t].astype(np.int64)
    assert np.array_equal(got.astype(np.int64), want)
    # and accumulating into an existing gradient adds it
    base = rng.integers(-5, 5, want.shape).astype(np.float32)
    got2 = o.embed_backward(lv, g, n_levels, dtable=base)
    assert np.array_equal(got2.astype(np.int64), want + base.astype(np.int64))


def test_embed_backward_adjoint_identity():
    # <dsum, A E> = <A^T dsum, E>: sum_t <g_t, s_t> = sum_rows <dE[row], E[row]>
    rng = np.random.default_rng(4)
    n, d = 200, 16
    lv = rng.integers(0, 16, (n, 80)).astype(np.uint8)
    E = rng.standard_normal((1280, d))
    g = rng.standard_normal((n, d)).astype(np.float32)
    rows = o.table_rows(lv)
    lhs = sum(float(np.dot(g[t].astype(np.float64), E[rows[t]].sum(axis=0))) for t in range(n))
    dE = o.embed_backward(lv, g)
    rhs = float(np.sum(dE.astype(np.float64) * E))
    assert abs(lhs - rhs) < 1e-4 * np.sum(np.abs(g)) * 10


def _one_row(terms):
    # one bin of one level: every token selects row 0
    g = np.array(terms, dtype=np.float32)[:, None]
    return np.zeros((len(terms), 1), dtype=np.uint8), g


def test_embed_backward_order_golden(golden_dir):
    with open(os.path.join(golden_dir, "embed_backward_order.json")) as f:
        c = json.load(f)
    lv, g = _one_row(c["order"]["terms"])
    assert o.embed_backward(lv, g, 1)[0, 0] == c["order"]["token_order"]
    # the hand-worked alternatives really are different numbers, so the pin
    # separates token order from reverse order and from adding halves first
    assert len({c["order"]["token_order"], c["order"]["reverse_order"], c["order"]["halves_first"]}) == 3
    lv, g = _one_row(c["accumulate"]["terms"])
    base = np.array([[c["accumulate"]["existing"]]], dtype=np.float32)
    assert o.embed_backward(lv, g, 1, dtable=base)[0, 0] == c["accumulate"]["result"]
    assert c["accumulate"]["result"] != c["accumulate"]["chained_from_existing"]
    lv, g = _one_row(c["signed_zero"]["terms"])
    got = o.embed_backward(lv, g, 1)[0, 0]
    assert got == 0.0 and int(np.signbit(got)) == c["signed_zero"]["result_sign_bit"]


def test_embed_backward_token_order_by_rows():
    # the same sums formed the other way round: for each row, its tokens
    # collected first, then added one by one as fp32 scalars; inputs drawn so
    # that order matters (large and small magnitudes mixed)
    rng = np.random.default_rng(7)
    n, d, n_bins, n_levels = 150, 3, 4, 3
    lv = rng.integers(0, n_levels, (n, n_bins)).astype(np.uint8)
    g = (rng.standard_normal((n, d)) * np.where(rng.random((n, d)) < 0.2, 1e7, 1.0)).astype(np.float32)
    got = o.embed_backward(lv, g, n_levels)
    for b in range(n_bins):
        for lev in range(n_levels):
            toks = [t for t in range(n) if lv[t, b] == lev]
            for c in range(d):
                acc = np.float32(0.0)
                for t in toks:
                    acc = np.float32(acc + g[t, c])
                assert got[n_levels * b + lev, c] == acc
    # a column subset is the same computation on those columns
    sub = o.embed_backward(lv, g, n_levels, cols=[2, 0])
    assert np.array_equal(sub, got[:, [2, 0]])


def test_embed_backward_untouched_rows_are_zero():
    lv = np.zeros((7, 80), dtype=np.uint8)
    g = np.ones((7, 4), dtype=np.float32)
    dE = o.embed_backward(lv, g)
    touched = 16 * np.arange(80)
    assert np.all(dE[touched] == 7.0)
    mask = np.ones(1280, bool)
    mask[touched] = False
    assert np.all(dE[mask] == 0) and not np.any(np.signbit(dE[mask]))
