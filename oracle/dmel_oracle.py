"""Plain CPU oracle for the dMel audio front end (numpy, fp64 / sequential fp32).

TEST INFRASTRUCTURE ONLY.  This module exists so that the HIP library can be
checked against an independent, obviously correct definition of what the
front end computes.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the C-ABI
library and its Python binding) never imports, calls or falls back to it, and
this module shares no code, tables or constants generator with the library.

Sources (the web pages this method is described on):

* "Inside Inkling: Audio Design", Part 1 - Modeling: 16 kHz mono audio becomes
  an 80-channel log-mel spectrogram with an 800-sample hop and a 1600-sample
  window; each of the 80 mel energies is quantized to one of 16 levels; the
  80 rows selected in an ``nn.Embedding(80*16 = 1280 -> 6144)`` table are
  summed into one 6144-d vector, optionally followed by RMSNorm.  The
  subsection "Why this is a reasonable bet" gives the rate constants
  (``audio_token_duration_s = 0.05``, ``window_size_multiplier = 2.0``,
  20 frames per second), the released config keys (``n_mel_bins: 80``,
  ``mel_vocab_size: 16``, clamp range ``dmel_min_value: -7.0`` /
  ``dmel_max_value: 2.0``) and says each mel bin owns its own block of 16
  table rows.
* Same page, Coda "What I don't know yet": the level mapping and the row
  layout are not documented; the config's -7.0 clamp minimum is said to win
  over a serving default of -1.5.
* "Why Thinking Machines Built Inkling Without a Vision Encoder": the rounding
  needs no training, so the front end is a fixed conversion.

Where the pages leave a step open, the reading taken is stated beside the step
(window shape, FFT size, power spectrum, HTK mel scale over 0-8000 Hz, natural
log with a 1e-10 floor, a uniform floor quantizer, causal framing, the row
layout ``16*bin + level``, and the RMSNorm form).

Precision: frames, FFT, power, mel, log and RMSNorm are fp64.  The embedding
sum is fp32, one IEEE round-to-nearest-even add per bin in bin order 0..79,
because that sequential fp32 sum *is* the definition of the embedding result.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Constants ("Inside Inkling: Audio Design", Part 1, "Why this is a
# reasonable bet": hop = 0.05 s * 16000 = 800, window = 2 * hop = 1600,
# n_mel_bins 80, mel_vocab_size 16, clamp [-7, 2]; the table width 6144 is
# the embedding's output dimension in the same section).
# ---------------------------------------------------------------------------
SAMPLE_RATE = 16000
HOP = 800
WINDOW = 1600
N_FFT = 1600               # reading: no zero padding -> 801 one-sided bins
N_BINS = N_FFT // 2 + 1    # 801
N_MELS = 80
N_LEVELS = 16
N_ROWS = N_MELS * N_LEVELS  # 1280
D_MODEL = 6144
CLAMP_MIN = -7.0
CLAMP_MAX = 2.0
LOG_FLOOR = 1e-10          # reading: natural log of max(M, 1e-10)
F_MIN = 0.0
F_MAX = SAMPLE_RATE / 2.0  # reading: filters span 0 .. 8000 Hz
RMS_EPS = 1e-6             # reading: RMSNorm epsilon


# ---------------------------------------------------------------------------
# Framing ("Inside Inkling: Audio Design", Part 1: hop 800, window 1600,
# no frame stacking or pooling -> 20 frames per second).
# Reading (causal framing): frame t covers samples [800 t - 800, 800 t + 800)
# of its clip; samples before 0 are the stream carry (or zeros).  A clip of N
# samples gives floor(N / 800) frames; the N mod 800 tail completes no frame.
# ---------------------------------------------------------------------------
def num_frames(n_samples: int) -> int:
    """Frames produced by a clip of ``n_samples`` samples (0 for a short clip)."""
    if n_samples < 0:
        raise ValueError("negative sample count")
    return int(n_samples) // HOP


def frame_signal(x: np.ndarray, carry: np.ndarray | None = None) -> np.ndarray:
    """Return the [T, 1600] fp64 frames of one clip.

    ``carry`` holds the 800 samples that precede the clip (zeros if None).
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    if carry is None:
        carry = np.zeros(HOP, dtype=np.float64)
    carry = np.asarray(carry, dtype=np.float64).reshape(-1)
    if carry.shape[0] != HOP:
        raise ValueError("carry must hold 800 samples")
    t_count = num_frames(x.shape[0])
    padded = np.concatenate([carry, x])
    frames = np.empty((t_count, WINDOW), dtype=np.float64)
    for t in range(t_count):
        # padded index p corresponds to clip sample p - 800
        frames[t] = padded[HOP * t: HOP * t + WINDOW]
    return frames


# ---------------------------------------------------------------------------
# Window and spectrum.  Readings: periodic Hann window of length 1600,
# n_fft = 1600 (801 bins), power |X|^2.
# ---------------------------------------------------------------------------
def hann_window() -> np.ndarray:
    n = np.arange(WINDOW, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * n / WINDOW)


def power_spectrum(frames: np.ndarray) -> np.ndarray:
    """|rfft(w * frame)|^2 for every frame: [T, 801] fp64."""
    frames = np.asarray(frames, dtype=np.float64)
    spec = np.fft.rfft(frames * hann_window()[None, :], n=N_FFT, axis=-1)
    return spec.real ** 2 + spec.imag ** 2


# ---------------------------------------------------------------------------
# Mel filterbank.  Reading: HTK mel scale m(f) = 2595 log10(1 + f / 700),
# 80 unit-peak triangles whose 82 edges are equally spaced in mel between
# 0 Hz and 8000 Hz, evaluated at the bin frequencies 10 k Hz (k = 0..800),
# no area normalisation.  The two outer edges are set to exactly 0 and 8000 Hz.
# ---------------------------------------------------------------------------
def hz_to_mel(f):
    return 2595.0 * np.log10(1.0 + np.asarray(f, dtype=np.float64) / 700.0)


def mel_to_hz(m):
    return 700.0 * (10.0 ** (np.asarray(m, dtype=np.float64) / 2595.0) - 1.0)


def mel_edges_hz(n_mels: int = N_MELS) -> np.ndarray:
    """The n_mels + 2 triangle edges in Hz (edges j, j+1, j+2 define filter j)."""
    if n_mels < 1:
        raise ValueError("n_mels must be positive")
    mels = np.linspace(hz_to_mel(F_MIN), hz_to_mel(F_MAX), n_mels + 2)
    hz = mel_to_hz(mels)
    hz[0] = F_MIN
    hz[-1] = F_MAX
    return hz


def bin_frequencies() -> np.ndarray:
    return np.arange(N_BINS, dtype=np.float64) * (SAMPLE_RATE / N_FFT)


def triangle(j: int, f, n_mels: int = N_MELS) -> np.ndarray:
    """Response of mel filter ``j`` (of ``n_mels``) at frequency ``f`` (Hz)."""
    e = mel_edges_hz(n_mels)
    f = np.asarray(f, dtype=np.float64)
    rise = (f - e[j]) / (e[j + 1] - e[j])
    fall = (e[j + 2] - f) / (e[j + 2] - e[j + 1])
    return np.maximum(0.0, np.minimum(rise, fall))


def mel_filterbank(n_mels: int = N_MELS) -> np.ndarray:
    """[n_mels, 801] fp64 filter weights H[j, k]."""
    freqs = bin_frequencies()
    return np.stack([triangle(j, freqs, n_mels) for j in range(n_mels)])


# ---------------------------------------------------------------------------
# Log-mel ("80-channel log-mel spectrogram"; reading: natural log of
# max(M, 1e-10)).
# ---------------------------------------------------------------------------
def log_mel_from_frames(frames: np.ndarray, n_mels: int = N_MELS) -> np.ndarray:
    power = power_spectrum(frames)
    mel = power @ mel_filterbank(n_mels).T
    return np.log(np.maximum(mel, LOG_FLOOR))


def log_mel(x: np.ndarray, carry: np.ndarray | None = None, n_mels: int = N_MELS) -> np.ndarray:
    """[T, n_mels] fp64 log-mel of one clip."""
    return log_mel_from_frames(frame_signal(x, carry), n_mels)


# ---------------------------------------------------------------------------
# Quantizer ("each of the 80 mel energies in a frame is quantized to one of
# 16 levels", clamp range [-7, 2]).  Reading: uniform floor over the clamp
# range, level = min(15, floor((clamp(l, -7, 2) + 7) * 16 / 9)).  The 15
# decision edges -7 + 9k/16 are exact binary fractions, and for fp32 or fp64
# inputs every step below is exact near an edge, so the level of a given
# value does not depend on the precision it is evaluated in.
#
# The same page's Coda says the serving code defaults the clamp minimum to
# -1.5 where the released config has -7, and the config names the level
# count (mel_vocab_size) and range (dmel_min_value, dmel_max_value) as
# parameters.  The parametric form is the same uniform floor over [lo, hi] in
# n_levels steps: level = min(n_levels - 1, floor((c - lo) * n_levels / (hi - lo))),
# c = clamp(l, lo, hi), decided as the number of edges
# e_k = lo + ((hi - lo) * k) / n_levels, k = 1 .. n_levels - 1, that c reaches,
# with e_k evaluated in fp64 in exactly that order.  When the edges are binary
# fractions (both page configurations) this is the exact floor formula; for
# other ranges it differs from it only within an fp64 rounding of an edge.
# ---------------------------------------------------------------------------
def level_edges(lo: float = CLAMP_MIN, hi: float = CLAMP_MAX, n_levels: int = N_LEVELS) -> np.ndarray:
    """The n_levels - 1 decision edges (value >= edge k -> level >= k)."""
    lo, hi = float(lo), float(hi)
    if not (np.isfinite(lo) and np.isfinite(hi) and lo < hi) or n_levels < 1:
        raise ValueError("need finite lo < hi and n_levels >= 1")
    k = np.arange(1, n_levels, dtype=np.float64)
    return lo + ((hi - lo) * k) / n_levels


def quantize(logmel: np.ndarray, lo: float = CLAMP_MIN, hi: float = CLAMP_MAX,
             n_levels: int = N_LEVELS) -> np.ndarray:
    """Levels of the reading floor((clamp(l, lo, hi) - lo) * n_levels / (hi - lo)), top folded.

    In exact arithmetic floor(y) >= k  <=>  y >= k  <=>  c >= lo + (hi - lo) k / n,
    so the level is the number of edges that the clamped value reaches.  The
    comparisons are exact; with the released edges (-7 + 9k/16, exact binary
    fractions) this evaluates the formula without any rounding, for fp32 and
    fp64 inputs alike.  (Evaluating (c + 7) * 16 / 9 in floating point
    instead can round a value one ulp below an edge onto the edge.)
    """
    if n_levels > 256:
        raise ValueError("levels are bytes: at most 256")
    l = np.asarray(logmel, dtype=np.float64)
    c = np.minimum(np.maximum(l, float(lo)), float(hi))
    return np.searchsorted(level_edges(lo, hi, n_levels), c, side="right").astype(np.uint8)


def levels(x: np.ndarray, carry: np.ndarray | None = None) -> np.ndarray:
    return quantize(log_mel(x, carry))


class Config:
    """A front-end configuration: the released config keys n_mel_bins,
    mel_vocab_size, dmel_min_value and dmel_max_value ("Why this is a
    reasonable bet"); the defaults are the released values."""

    def __init__(self, n_mel_bins: int = N_MELS, mel_vocab_size: int = N_LEVELS,
                 min_value: float = CLAMP_MIN, max_value: float = CLAMP_MAX):
        self.n_mel_bins = int(n_mel_bins)
        self.mel_vocab_size = int(mel_vocab_size)
        self.min_value = float(min_value)
        self.max_value = float(max_value)


def levels_cfg(x: np.ndarray, cfg: Config, carry: np.ndarray | None = None):
    """(log-mel [T, n_mel_bins], levels [T, n_mel_bins]) of one clip under cfg."""
    lm = log_mel(x, carry, cfg.n_mel_bins)
    return lm, quantize(lm, cfg.min_value, cfg.max_value, cfg.mel_vocab_size)


# ---------------------------------------------------------------------------
# bfloat16 helpers (the table is bf16; outputs are rounded to bf16 with
# round-to-nearest-even).  bf16 is the top half of an fp32 bit pattern.
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bits, nearest-even (finite inputs only)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bits, nearest-even, in one rounding.

    Valid for finite values whose bf16 result is a normal number.  The fp64
    fraction has 52 bits and bf16 keeps the top 7, so the rounding happens at
    fraction bit 45; the rounded fp64 value is then exactly an fp32 value whose
    top half is the bf16 pattern.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = x.view(np.uint64)
    half = np.uint64((1 << 44) - 1)
    r = (u + half + ((u >> np.uint64(45)) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
    y = r.view(np.float64)
    mag = np.abs(y)
    if np.any((mag != 0) & ((mag < 2.0 ** -126) | (mag > 3.3e38))):
        raise ValueError("value outside the normal bf16 range")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Embedding bag ("A frame's 80 rows are summed into one 6144-dimensional
# vector"; "each mel bin owns its own block of 16 rows").  Reading: row
# r_j = 16 j + L_j; fp32 accumulation, s = E[r_0], then s = fl32(s + E[r_j])
# for j = 1..79, in that order.  With another mel_vocab_size V the block of a
# bin has V rows (r_j = V j + L_j) and the table n_bins * V rows, as in the
# config's nn.Embedding(n_mel_bins * mel_vocab_size -> d).
# ---------------------------------------------------------------------------
def table_rows(lv: np.ndarray, n_levels: int = N_LEVELS) -> np.ndarray:
    lv = np.asarray(lv).astype(np.int64)
    if lv.ndim != 2:
        raise ValueError("levels must be [n, n_bins]")
    if np.any(lv >= n_levels):
        raise ValueError("level out of range")
    return n_levels * np.arange(lv.shape[1], dtype=np.int64)[None, :] + lv


def embed_sum(lv: np.ndarray, table_bits: np.ndarray, n_levels: int = N_LEVELS) -> np.ndarray:
    """Sequential fp32 bag-of-bins sum: [n, d] fp32."""
    table = bf16_to_f32(table_bits)
    rows = table_rows(lv, n_levels)
    s = table[rows[:, 0]].astype(np.float32, copy=True)
    for j in range(1, rows.shape[1]):
        s = (s + table[rows[:, j]]).astype(np.float32, copy=False)
    return s


def rms_norm(s: np.ndarray, weight: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Reading of the optional RMSNorm: y = s * w / sqrt(mean(s^2) + eps), fp64."""
    s64 = np.asarray(s, dtype=np.float64)
    w64 = np.asarray(weight, dtype=np.float64)
    ms = np.mean(s64 * s64, axis=-1, keepdims=True)
    return s64 * w64[None, :] / np.sqrt(ms + eps)


def embed(lv: np.ndarray, table_bits: np.ndarray, rms_weight: np.ndarray | None = None,
          eps: float = RMS_EPS, out_dtype: str = "bf16", n_levels: int = N_LEVELS):
    """Audio tokens from levels.

    Returns ``(out, exact)``: ``out`` is bf16 bits (uint16) or fp32; ``exact``
    is the unrounded value (the fp32 sum without RMSNorm, the fp64 RMSNorm
    output with it) that tolerance checks use.
    """
    s = embed_sum(lv, table_bits, n_levels)
    if rms_weight is None:
        exact = s
        out = f32_to_bf16(s) if out_dtype == "bf16" else s.copy()
    else:
        exact = rms_norm(s, rms_weight, eps)
        out = f64_to_bf16(exact) if out_dtype == "bf16" else exact.astype(np.float32)
    return out, exact


def forward(x: np.ndarray, table_bits: np.ndarray, rms_weight=None, eps: float = RMS_EPS,
            out_dtype: str = "bf16", carry=None, cfg: Config | None = None):
    """One clip end to end: audio -> log-mel -> levels -> tokens (cfg: None = released)."""
    cfg = cfg or Config()
    lm, lv = levels_cfg(x, cfg, carry)
    out, exact = embed(lv, table_bits, rms_weight, eps, out_dtype, n_levels=cfg.mel_vocab_size)
    return lm, lv, out, exact


# ---------------------------------------------------------------------------
# Backward (training the front end jointly with the model: "Inside Inkling:
# Audio Design", Coda, the front ends are frozen in post-training and training
# them is experimental).  The pages give no backward;
# it is the derivative of the forward above.
#
# RMSNorm: y = s * r * w with r = 1 / sqrt(mean(s^2) + eps), so for an
# upstream gradient dy
#     ds = r * (w * dy) - (r^3 / D) * (sum_c w_c dy_c s_c) * s
#     dw = sum_t dy_t * s_t * r_t
# (evaluated in fp64 from the fp32 sum s).
#
# Embedding bag: dE[row] = sum of ds_t over the (t, j) with row r_tj = row.
# Reading of the summation order (the pages give none): the plain definition,
# each row's gradients added in increasing token order, one fp32 add per
# selecting token, starting from +0 (the table gradient is a zero tensor that
# every token adds its gradient into, token by token).  When accumulating
# into an existing gradient G, the result is fl32(G + S) with S that sum (an
# existing gradient plus a freshly computed one, as an optimizer's gradient
# buffer receives it).
# ---------------------------------------------------------------------------


def rms_backward(lv: np.ndarray, table_bits: np.ndarray, weight, dy, eps: float = RMS_EPS,
                 n_levels: int = N_LEVELS):
    """(ds fp64 [n, d], dw fp64 [d], s fp32 [n, d], r fp64 [n]) for levels lv and upstream dy."""
    s = embed_sum(lv, table_bits, n_levels)
    ds, dw, r = rms_backward_from_sum(s, weight, dy, eps)
    return ds, dw, s, r


def rms_backward_from_sum(s, weight, dy, eps: float = RMS_EPS):
    """(ds, dw, r) of y = s * w / sqrt(mean(s^2) + eps) for rows s, in fp64."""
    s64 = np.asarray(s, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    g = np.asarray(dy, dtype=np.float64)
    d = s64.shape[1]
    r = 1.0 / np.sqrt(np.mean(s64 * s64, axis=1) + eps)
    dot = np.sum(w[None, :] * g * s64, axis=1)
    ds = r[:, None] * (w[None, :] * g) - (r ** 3 / d)[:, None] * dot[:, None] * s64
    dw = np.sum(g * s64 * r[:, None], axis=0)
    return ds, dw, r


def embed_backward(lv: np.ndarray, dsum, n_levels: int = N_LEVELS, dtable=None, cols=None):
    """fp32 [n_bins * n_levels, d] gradient of the table, each row summed in
    token order from +0 (see above).

    dsum: [n, d] gradient with respect to the fp32 sum (fp32 values, or bf16
    values given as fp32).  dtable: existing gradient to accumulate into.
    cols: optional column indices; only those columns are computed (the
    result is then [rows, len(cols)]) - columns are independent sums, so this
    changes nothing but the cost."""
    g = np.asarray(dsum, dtype=np.float32)
    if cols is not None:
        g = g[:, np.asarray(cols)]
    rows = table_rows(np.minimum(np.asarray(lv), n_levels - 1), n_levels)
    n, n_bins = rows.shape
    d = g.shape[1]
    total = np.zeros((n_bins * n_levels, d), dtype=np.float32)
    for t in range(n):
        # the token's rows are distinct (one per bin): one fp32 add each, and
        # the tokens arrive in order
        total[rows[t]] = total[rows[t]] + g[t][None, :]
    if dtable is not None:
        base = np.asarray(dtable, dtype=np.float32)
        if cols is not None:
            base = base[:, np.asarray(cols)]
        total = base + total
    return total


# ---------------------------------------------------------------------------
# Serving-path placement ("Where audio touches the serving path": one audio
# item is a sentinel expanded into f frame positions).  An interleaved
# sequence is a list of segments in order; a text segment contributes one
# output row per id, copied from the text table; an audio segment contributes
# its clip's tokens in frame order.
# ---------------------------------------------------------------------------
def interleave(segments, table_bits, text_table_bits):
    """segments: list of ("text", ids) or ("audio", samples).  Returns bf16 rows."""
    rows = []
    for kind, payload in segments:
        if kind == "text":
            ids = np.asarray(payload, dtype=np.int64)
            rows.append(np.asarray(text_table_bits)[ids])
        elif kind == "audio":
            _, _, out, _ = forward(payload, table_bits)
            rows.append(out)
        else:
            raise ValueError(kind)
    d = np.asarray(table_bits).shape[1]
    if not rows:
        return np.zeros((0, d), dtype=np.uint16)
    return np.concatenate(rows, axis=0)
