"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each check compares the oracle with something other than itself: a constant
the pages state, a closed form, an invariant, a textbook special case, or
brute force on a tiny input.  A plausible slip in the oracle (a dropped term,
a wrong sign, index or operand order) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import dmel_oracle as o


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Page constants
# ---------------------------------------------------------------------------
def test_page_constants(golden_dir):
    c = _load(golden_dir, "page_constants.json")
    assert o.SAMPLE_RATE == c["sample_rate_hz"]["value"]
    assert o.HOP == round(c["audio_token_duration_s"]["value"] * c["sample_rate_hz"]["value"])
    assert o.HOP == c["hop_samples"]["value"]
    assert o.WINDOW == round(c["window_size_multiplier"]["value"] * o.HOP) == c["window_samples"]["value"]
    assert o.N_MELS == c["n_mel_bins"]["value"]
    assert o.N_LEVELS == c["mel_vocab_size"]["value"]
    assert o.N_ROWS == c["table_rows"]["value"] == o.N_MELS * o.N_LEVELS
    assert o.D_MODEL == c["d_model"]["value"]
    assert o.CLAMP_MIN == c["dmel_min_value"]["value"]
    assert o.CLAMP_MAX == c["dmel_max_value"]["value"]
    params = o.N_ROWS * o.D_MODEL
    assert params == 7_864_320
    assert round(params / 1e6, 1) == c["table_params_approx_millions"]["value"]


def test_frame_rate_pins(golden_dir):
    c = _load(golden_dir, "page_constants.json")
    sr = c["sample_rate_hz"]["value"]
    # 1 s of audio -> 20 tokens; 20 minutes -> 24k tokens
    assert o.num_frames(sr) == c["tokens_per_second"]["value"]
    assert o.num_frames(c["max_clip_minutes"]["value"] * 60 * sr) == c["tokens_per_20_min_clip"]["value"]
    # a short clip completes no frame; the tail past the last full hop is dropped
    assert o.num_frames(0) == 0
    assert o.num_frames(799) == 0
    assert o.num_frames(800) == 1
    assert o.num_frames(1599) == 1
    x = np.arange(2500, dtype=np.float64)
    fr = o.frame_signal(x)
    assert fr.shape == (3, 1600)
    # frame t = samples [800 t - 800, 800 t + 800), zeros before the clip
    assert np.all(fr[0, :800] == 0) and np.array_equal(fr[0, 800:], x[:800])
    assert np.array_equal(fr[2], x[800:2400])
    carry = -np.arange(1, 801, dtype=np.float64)
    fc = o.frame_signal(x, carry)
    assert np.array_equal(fc[0, :800], carry) and np.array_equal(fc[1:], fr[1:])


# ---------------------------------------------------------------------------
# Window and FFT
# ---------------------------------------------------------------------------
def test_hann_closed_forms():
    w = o.hann_window()
    assert w.shape == (1600,)
    assert abs(w.sum() - 800.0) < 1e-9
    assert abs((w * w).sum() - 600.0) < 1e-9
    assert w[0] == 0.0 and abs(w[800] - 1.0) < 1e-15
    # periodic: symmetric about n = 800 with w[n] = w[1600 - n]
    assert np.allclose(w[1:], w[1:][::-1], atol=1e-15)
    W = np.fft.fft(w)
    assert abs(W[0] - 800) < 1e-9 and abs(W[1] + 400) < 1e-9 and abs(W[-1] + 400) < 1e-9
    assert np.max(np.abs(W[2:-1])) < 1e-9


def test_power_matches_direct_dft():
    rng = np.random.default_rng(7)
    frames = rng.standard_normal((3, 1600))
    w = o.hann_window()
    n = np.arange(1600)
    k = np.arange(801)
    # brute force O(N^2) DFT, no FFT involved
    basis = np.exp(-2j * np.pi * np.outer(k, n) / 1600.0)
    direct = np.abs((frames * w) @ basis.T) ** 2
    got = o.power_spectrum(frames)
    assert got.shape == (3, 801)
    assert np.max(np.abs(got - direct) / (np.abs(direct) + 1e-9 * direct.max())) < 1e-9


def test_parseval():
    rng = np.random.default_rng(8)
    frames = rng.standard_normal((4, 1600))
    p = o.power_spectrum(frames)
    c = np.full(801, 2.0)
    c[0] = c[800] = 1.0
    lhs = (p * c).sum(axis=1)
    rhs = 1600.0 * ((frames * o.hann_window()) ** 2).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-12)


def test_constant_input_spectrum():
    a = 0.37
    p = o.power_spectrum(np.full((1, 1600), a))[0]
    assert abs(p[0] - 640000 * a * a) < 1e-6
    assert abs(p[1] - 160000 * a * a) < 1e-6
    assert np.max(np.abs(p[2:])) < 1e-12


def test_bin_centred_cosine_closed_form():
    amp, m, phi = 0.3, 100, 0.7
    n = np.arange(1600)
    x = amp * np.cos(2 * np.pi * m * n / 1600 + phi)
    p = o.power_spectrum(x[None, :])[0]
    assert abs(p[m] - (400 * amp) ** 2) < 1e-6            # 14400
    assert abs(p[m - 1] - (200 * amp) ** 2) < 1e-6        # 3600
    assert abs(p[m + 1] - (200 * amp) ** 2) < 1e-6
    mask = np.ones(801, bool)
    mask[m - 1:m + 2] = False
    assert np.max(np.abs(p[mask])) < 1e-8
    # log-mel of a steady tone, for any full frame (t >= 1), in closed form
    sig = amp * np.cos(2 * np.pi * m * np.arange(4000) / 1600 + phi)
    lm = o.log_mel(sig)
    H = o.mel_filterbank()
    want = np.log(np.maximum(H[:, m] * (400 * amp) ** 2 + (H[:, m - 1] + H[:, m + 1]) * (200 * amp) ** 2, 1e-10))
    for t in range(1, lm.shape[0]):
        assert np.max(np.abs(lm[t] - want)) < 1e-8


# ---------------------------------------------------------------------------
# Mel filterbank
# ---------------------------------------------------------------------------
def test_htk_mel_scale_textbook_point():
    # the HTK mel scale is built so that 1000 Hz maps to ~1000 mel
    assert abs(o.hz_to_mel(1000.0) - 1000.0) < 0.05
    assert abs(o.mel_to_hz(o.hz_to_mel(1234.5)) - 1234.5) < 1e-9
    assert o.hz_to_mel(0.0) == 0.0


def test_filterbank_structure():
    H = o.mel_filterbank()
    e = o.mel_edges_hz()
    f = o.bin_frequencies()
    assert H.shape == (80, 801)
    assert e[0] == 0.0 and e[-1] == 8000.0 and np.all(np.diff(e) > 0)
    # edges equally spaced in mel
    dm = np.diff(o.hz_to_mel(e))
    assert np.allclose(dm, dm[0], rtol=1e-9)
    # unit-peak triangles, every filter non-empty, weights in [0, 1]
    assert np.all(H >= 0) and np.all(H <= 1)
    assert np.all((H > 0).sum(axis=1) >= 1)
    for j in (0, 17, 79):
        assert abs(o.triangle(j, e[j + 1]) - 1.0) < 1e-12
        assert o.triangle(j, e[j]) == 0.0 and o.triangle(j, e[j + 2]) == 0.0
    # partition of unity between the first and last centre
    inner = (f >= e[1]) & (f <= e[80])
    assert np.max(np.abs(H[:, inner].sum(axis=0) - 1.0)) < 1e-12
    # the bin at Nyquist gets no weight (outer edge exactly 8000 Hz)
    assert H[:, 800].max() == 0.0
    # filter j only covers bins strictly between its outer edges
    for j in range(80):
        nz = np.nonzero(H[j])[0]
        assert f[nz].min() > e[j] and f[nz].max() < e[j + 2]


def test_tone_peaks_in_its_band():
    t = np.arange(16000) / 16000.0
    H = o.mel_filterbank()
    e = o.mel_edges_hz()
    for f0 in (150.0, 440.0, 1000.0, 2500.0, 6000.0):
        lm = o.log_mel(0.3 * np.sin(2 * np.pi * f0 * t))
        best = int(np.argmax(lm[5]))
        resp = np.array([o.triangle(j, f0) for j in range(80)])
        candidates = set(np.nonzero(resp >= resp.max() - 1e-9)[0].tolist())
        # where two triangles cross, accept either neighbour
        k = int(round(f0 / 10.0))
        for kk in (k - 1, k, k + 1):
            candidates |= set(np.nonzero(H[:, kk] == H[:, kk].max())[0].tolist())
        assert best in candidates, (f0, best, candidates)
        assert e[best] < f0 < e[best + 2]


# ---------------------------------------------------------------------------
# Floor, clamp and levels
# ---------------------------------------------------------------------------
def test_silence_floor_and_level_zero():
    lm = o.log_mel(np.zeros(4000))
    assert lm.shape == (5, 80)
    assert np.all(lm == np.log(1e-10))
    assert abs(lm[0, 0] - (-23.025850929940457)) < 1e-12
    assert np.all(o.quantize(lm) == 0)


def test_quantizer_golden(golden_dir):
    c = _load(golden_dir, "quantizer_levels.json")
    xs = np.array([v for v, _ in c["cases"]])
    want = np.array([lv for _, lv in c["cases"]])
    assert np.array_equal(o.quantize(xs), want)


def test_quantizer_edges_bruteforce():
    edges = o.level_edges()
    assert edges.shape == (15,)
    assert np.allclose(np.diff(edges), 9.0 / 16.0)
    for k, e in enumerate(edges, start=1):
        assert o.quantize(np.array([e]))[0] == k
        assert o.quantize(np.array([np.nextafter(e, -np.inf)]))[0] == k - 1
        # fp32 inputs decide exactly like fp64 ones
        e32 = np.float32(e)
        assert float(e32) == e
        assert o.quantize(np.array([np.nextafter(e32, np.float32(-np.inf))], dtype=np.float32))[0] == k - 1
    grid = np.linspace(-10, 5, 200001)
    q = o.quantize(grid)
    assert np.all(np.diff(q.astype(int)) >= 0)
    assert q.min() == 0 and q.max() == 15
    # every level spans the same width 9/16 inside the clamp range
    counts = np.bincount(q[(grid >= -7) & (grid < 2)], minlength=16)
    assert counts.min() > 0 and (counts.max() - counts.min()) <= 2


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------
def test_bf16_rounding_golden(golden_dir):
    c = _load(golden_dir, "bf16_rounding.json")
    f = np.array([int(x["f32_hex"], 16) for x in c["cases"]], dtype=np.uint32).view(np.float32)
    want = np.array([int(x["bf16_hex"], 16) for x in c["cases"]], dtype=np.uint16)
    assert np.array_equal(o.f32_to_bf16(f), want)
    # widening is exact
    assert np.array_equal(o.f32_to_bf16(o.bf16_to_f32(want)), want)


def test_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000) * 10.0 ** rng.uniform(-3, 3, 20000)
    got = o.f64_to_bf16(x)
    # brute force: nearest of the two bf16 neighbours, ties to even
    lo = o.f32_to_bf16(x.astype(np.float32))
    for i in range(0, 20000, 7):
        cands = [int(lo[i]) - 1, int(lo[i]), int(lo[i]) + 1]
        vals = [float(o.bf16_to_f32(np.array([c], np.uint16))[0]) for c in cands]
        d = [abs(v - x[i]) for v in vals]
        best = min(range(3), key=lambda q: (d[q], cands[q] & 1))
        assert got[i] == cands[best]
    # an exact fp64 tie that fp32 rounding would break: 1 + 2^-8 + 2^-40
    assert o.f64_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert o.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80


# ---------------------------------------------------------------------------
# Embedding sum
# ---------------------------------------------------------------------------
def test_fixed_order_golden(golden_dir):
    c = _load(golden_dir, "fixed_order.json")
    d = len(c["columns"])
    table = np.full((1280, d), np.float32(c["poison"]), dtype=np.float32)
    L = np.array([(7 * j + 3) % 16 for j in range(80)])
    r = 16 * np.arange(80) + L
    col = np.zeros((80, d), dtype=np.float64)
    col[:, 0] = 2.0 ** -24
    col[0, 0] = 1.0
    col[:, 1] = 0.0
    col[0, 1], col[1, 1], col[2, 1] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    col[:, 2] = 0.0
    col[0, 2], col[1, 2] = 1.0, 1.5 * 2.0 ** -24
    col[:, 3] = np.arange(80)
    col[:, 4] = -0.0
    table[r] = col.astype(np.float32)
    bits = o.f32_to_bf16(table)
    assert np.array_equal(o.bf16_to_f32(bits), table)  # every value is exact in bf16
    s = o.embed_sum(L[None, :], bits)[0]
    want = np.array([int(x["expect_f32_hex"], 16) for x in c["columns"]], dtype=np.uint32)
    assert np.array_equal(s.view(np.uint32), want)
    out, _ = o.embed(L[None, :], bits)
    want16 = np.array([int(x["expect_bf16_hex"], 16) for x in c["columns"]], dtype=np.uint16)
    assert np.array_equal(out[0], want16)


def test_integer_table_indexing_bruteforce():
    rng = np.random.default_rng(11)
    table = rng.integers(-8, 9, size=(1280, 24)).astype(np.float32)
    bits = o.f32_to_bf16(table)
    lv = rng.integers(0, 16, size=(6, 80)).astype(np.uint8)
    s = o.embed_sum(lv, bits)
    for t in range(6):
        ref = [0] * 24
        for j in range(80):
            row = j * 16 + int(lv[t, j])
            for c in range(24):
                ref[c] += int(table[row, c])
        assert np.array_equal(s[t], np.array(ref, dtype=np.float32))
    zero = np.zeros((1, 80), np.uint8)
    assert np.array_equal(o.embed_sum(zero, bits)[0], table[0::16].sum(axis=0))


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(12)
    s = rng.standard_normal((5, 64)).astype(np.float32)
    w1 = np.ones(64)
    y = o.rms_norm(s, w1, 1e-6)
    m = np.mean(s.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(y ** 2, axis=1), m / (m + 1e-6), rtol=1e-12)
    w = rng.uniform(0.5, 2.0, 64)
    assert np.allclose(o.rms_norm(s, w, 1e-6), y * w[None, :], rtol=1e-12)
    # scale invariance (eps small against the mean square)
    assert np.allclose(o.rms_norm(8.0 * s, w1, 1e-12), o.rms_norm(s, w1, 1e-12), rtol=1e-9)
    assert np.all(np.sign(y) == np.sign(s))


# ---------------------------------------------------------------------------
# End to end
# ---------------------------------------------------------------------------
def test_streaming_equals_batch():
    rng = np.random.default_rng(13)
    x = rng.standard_normal(800 * 7) * 0.1
    batch = o.levels(x)
    prev = np.zeros(800)
    for s in range(7):
        hop = x[800 * s: 800 * (s + 1)]
        step = o.levels(hop, carry=prev)
        assert step.shape == (1, 80)
        assert np.array_equal(step[0], batch[s])
        prev = hop


def test_forward_shapes_and_silence():
    rng = np.random.default_rng(14)
    table = o.f32_to_bf16(rng.standard_normal((1280, 32)).astype(np.float32) * 0.02)
    x = np.zeros(16000)
    x[4000:] = rng.standard_normal(12000) * 0.1
    lm, lv, out, exact = o.forward(x, table)
    assert lm.shape == (20, 80) and lv.shape == (20, 80) and out.shape == (20, 32)
    # frames 0..4 only see the silent first 0.25 s
    assert np.all(lv[:5] == 0)
    silent_token = o.embed_sum(np.zeros((1, 80), np.uint8), table)[0]
    assert np.array_equal(exact[0], silent_token)


def test_interleave_order():
    rng = np.random.default_rng(15)
    table = o.f32_to_bf16(rng.standard_normal((1280, 8)).astype(np.float32) * 0.02)
    text = o.f32_to_bf16(rng.standard_normal((50, 8)).astype(np.float32))
    audio = rng.standard_normal(800 * 3) * 0.1
    segs = [("text", [3, 4]), ("audio", audio), ("text", [49])]
    out = o.interleave(segs, table, text)
    assert out.shape == (2 + 3 + 1, 8)
    assert np.array_equal(out[0], text[3]) and np.array_equal(out[5], text[49])
    assert np.array_equal(out[2:5], o.forward(audio, table)[2])
