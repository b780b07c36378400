"""Seeded synthetic inputs for the dMel front end.

This module only draws signals, tables and layouts.  It holds none of the
front end's arithmetic (no framing, spectrum, mel, quantizer or embedding
step), so both the HIP path and the CPU oracle may consume what it makes.

The pages evaluate on public speech sets that are not available here; these
signals stand in for speech with the shapes, rates and value ranges of the
workloads the front end is run on (16 kHz mono fp32 audio, a 1280 x 6144
bf16 table drawn from N(0, 0.02)).

Random parameters (tone frequencies, syllable lengths, burst placement ...)
come from ``numpy.random.default_rng(seed)`` and are device independent.
Per-sample noise for the large workloads is drawn with a seeded
``torch.Generator`` on the device the audio is made on; the oracle always
consumes the exact arrays that were handed to the GPU, copied back.
"""

from __future__ import annotations

import math

import numpy as np
import torch

SAMPLE_RATE = 16000
HOP = 800
N_ROWS = 1280
D_MODEL = 6144


# ---------------------------------------------------------------------------
# Tables
# ---------------------------------------------------------------------------
def table_bf16(seed: int = 1234, rows: int = N_ROWS, d_model: int = D_MODEL,
               std: float = 0.02, device="cpu") -> torch.Tensor:
    """[rows, d_model] bf16 table ~ N(0, std), returned as its uint16 bit pattern
    in an int16 tensor (``.view(torch.bfloat16)`` gives the values)."""
    if str(device) == "cpu" or rows * d_model <= 64 * 1024 * 1024:
        rng = np.random.default_rng(seed)
        vals = torch.from_numpy((rng.standard_normal((rows, d_model)) * std).astype(np.float32))
        t = vals.to(torch.bfloat16).view(torch.int16)
        return t.to(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((rows, d_model), dtype=torch.bfloat16, device=device)
    chunk = max(1, (64 * 1024 * 1024) // d_model)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = (torch.randn((r1 - r0, d_model), generator=g, device=device) * std).to(torch.bfloat16)
    return out.view(torch.int16)


def integer_table(seed: int, rows: int = N_ROWS, d_model: int = D_MODEL, lo: int = -8, hi: int = 8) -> torch.Tensor:
    """Table of small integers (exact in bf16 and in any fp32 sum of 80 rows)."""
    rng = np.random.default_rng(seed)
    vals = torch.from_numpy(rng.integers(lo, hi + 1, size=(rows, d_model)).astype(np.float32))
    return vals.to(torch.bfloat16).view(torch.int16)


# ---------------------------------------------------------------------------
# Config 1: 1 s, three sinusoids + N(0, 0.01) noise, first 0.25 s silent.
# ---------------------------------------------------------------------------
def tones_clip(seed: int = 0, n_samples: int = SAMPLE_RATE, n_tones: int = 3, amp: float = 0.3,
               noise: float = 0.01, silent_samples: int = SAMPLE_RATE // 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    freqs = rng.uniform(100.0, 6000.0, size=n_tones)
    n = np.arange(n_samples, dtype=np.float64)
    x = np.zeros(n_samples, dtype=np.float64)
    for f in freqs:
        x += amp * np.sin(2.0 * np.pi * f * n / SAMPLE_RATE)
    x += rng.normal(0.0, noise, size=n_samples)
    x[:silent_samples] = 0.0
    return x.astype(np.float32)


# ---------------------------------------------------------------------------
# Config 2 / 4 signal model: pink noise (RMS 0.1) + rectangular tone bursts
# (50-500 ms, 100-6000 Hz, amplitude 0.1-0.5, 1.5 per second), peak-limited
# to |x| <= 1, then non-overlapping silent spans of 0.2-1.0 s until at least
# 10% of the samples are exactly zero.
# ---------------------------------------------------------------------------
def _silence_spans(rng: np.random.Generator, n_samples: int, frac: float = 0.10):
    spans = []
    silent = 0
    target = int(math.ceil(frac * n_samples))
    tries = 0
    while silent < target and tries < 10000:
        tries += 1
        ln = int(rng.uniform(0.2, 1.0) * SAMPLE_RATE)
        ln = min(ln, n_samples)
        st = int(rng.integers(0, max(1, n_samples - ln + 1)))
        if any(st < b and a < st + ln for a, b in spans):
            continue
        spans.append((st, st + ln))
        silent += ln
    return spans


def bursts_clips(seed: int, n_clips: int, n_samples: int, device="cpu") -> torch.Tensor:
    """[n_clips, n_samples] fp32 audio of the pink-noise + tone-burst model."""
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    seconds = n_samples / SAMPLE_RATE
    n_bursts = int(math.ceil(1.5 * seconds))
    out = torch.empty((n_clips, n_samples), dtype=torch.float32, device=device)
    # burst parameters for every clip, drawn up front (device independent)
    b_start = (rng.uniform(0.0, seconds, size=(n_clips, n_bursts)) * SAMPLE_RATE).astype(np.int64)
    b_len = (rng.uniform(0.05, 0.5, size=(n_clips, n_bursts)) * SAMPLE_RATE).astype(np.int64)
    b_freq = rng.uniform(100.0, 6000.0, size=(n_clips, n_bursts))
    b_amp = rng.uniform(0.1, 0.5, size=(n_clips, n_bursts))
    spans = [_silence_spans(rng, n_samples) for _ in range(n_clips)]
    max_len = int(0.5 * SAMPLE_RATE) + 1
    n_rfft = n_samples // 2 + 1
    k = torch.arange(n_rfft, device=device, dtype=torch.float64)
    shape = torch.where(k > 0, 1.0 / torch.sqrt(torch.clamp(k, min=1.0)), torch.zeros_like(k))
    chunk = max(1, int(2 ** 26 // max(1, n_samples)))
    for c0 in range(0, n_clips, chunk):
        c1 = min(n_clips, c0 + chunk)
        nc = c1 - c0
        white = torch.randn((nc, n_samples), generator=g, device=device, dtype=torch.float32)
        spec = torch.fft.rfft(white.double(), dim=-1) * shape[None, :]
        pink = torch.fft.irfft(spec, n=n_samples, dim=-1)
        rms = torch.sqrt(torch.mean(pink * pink, dim=-1, keepdim=True))
        x = (pink * (0.1 / rms)).float()
        # tone bursts: one scatter-add per burst slot, vectorised over clips
        ar = torch.arange(max_len, device=device)
        for b in range(n_bursts):
            st = torch.from_numpy(b_start[c0:c1, b]).to(device)
            ln = torch.from_numpy(b_len[c0:c1, b]).to(device)
            fr = torch.from_numpy(b_freq[c0:c1, b]).to(device)
            am = torch.from_numpy(b_amp[c0:c1, b]).to(device)
            idx = st[:, None] + ar[None, :]
            keep = (ar[None, :] < ln[:, None]) & (idx < n_samples)
            tone = am[:, None] * torch.sin(2.0 * math.pi * fr[:, None] * idx.double() / SAMPLE_RATE)
            tone = torch.where(keep, tone, torch.zeros_like(tone)).float()
            x.scatter_add_(1, torch.clamp(idx, max=n_samples - 1), tone)
        peak = torch.amax(torch.abs(x), dim=-1, keepdim=True)
        x = torch.where(peak > 1.0, x / peak, x)
        # silent spans: exact zeros
        rows, cols, vals = [], [], []
        for ci in range(nc):
            for a, b in spans[c0 + ci]:
                rows += [ci, ci]
                cols += [a, b]
                vals += [1, -1]
        mark = torch.zeros((nc, n_samples + 1), dtype=torch.int32, device=device)
        if rows:
            mark.index_put_((torch.tensor(rows, device=device), torch.tensor(cols, device=device)),
                            torch.tensor(vals, dtype=torch.int32, device=device), accumulate=True)
        silent = torch.cumsum(mark, dim=-1)[:, :n_samples] > 0
        x = torch.where(silent, torch.zeros_like(x), x)
        out[c0:c1] = x
    return out


# ---------------------------------------------------------------------------
# Config 3 / 5 signal model ("speech-like"): consecutive syllables of
# 0.1-0.4 s; each a harmonic stack with constant f0 ~ U[80, 300] Hz,
# harmonics h = 1..floor(7900 / f0) with amplitude 1/h and random phase,
# scaled to peak 0.5, shaped by a sin^2 envelope over the syllable, plus
# N(0, 0.02) noise.
# ---------------------------------------------------------------------------
MAX_HARMONICS = 7900 // 80  # 98


def speech_clips(seed: int, lengths, device="cpu") -> torch.Tensor:
    """Concatenated speech-like audio for clips of the given sample lengths.

    Returns a flat fp32 tensor of ``sum(lengths)`` samples (clip after clip).
    """
    lengths = [int(v) for v in lengths]
    total = int(sum(lengths))
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    # syllable boundaries per clip (global sample positions)
    starts, lens, f0s = [], [], []
    pos = 0
    for ln in lengths:
        t = 0
        while t < ln:
            sl = int(rng.uniform(0.1, 0.4) * SAMPLE_RATE)
            sl = max(1, min(sl, ln - t))
            starts.append(pos + t)
            lens.append(sl)
            f0s.append(rng.uniform(80.0, 300.0))
            t += sl
        pos += ln
    n_syl = len(starts)
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(n_syl, MAX_HARMONICS))
    starts_t = torch.tensor(starts, dtype=torch.int64, device=device)
    lens_t = torch.tensor(lens, dtype=torch.int64, device=device)
    f0_t = torch.tensor(f0s, dtype=torch.float64, device=device)
    nh_t = torch.floor(7900.0 / f0_t).to(torch.int64)
    ph_t = torch.tensor(phases, dtype=torch.float32, device=device)
    out = torch.empty(total, dtype=torch.float32, device=device)
    chunk = 1 << 21
    stack = torch.empty(total, dtype=torch.float32, device=device)
    for s0 in range(0, total, chunk):
        s1 = min(total, s0 + chunk)
        n = torch.arange(s0, s1, device=device, dtype=torch.int64)
        sid = torch.searchsorted(starts_t, n, right=True) - 1
        tau = (n - starts_t[sid]).double()
        theta = (2.0 * math.pi / SAMPLE_RATE) * f0_t[sid] * tau
        theta = torch.remainder(theta, 2.0 * math.pi).float()
        acc = torch.zeros(s1 - s0, dtype=torch.float32, device=device)
        nh = nh_t[sid]
        for h in range(1, MAX_HARMONICS + 1):
            term = torch.sin(h * theta + ph_t[sid, h - 1]) / h
            acc += torch.where(nh >= h, term, torch.zeros_like(term))
        stack[s0:s1] = acc
    # scale every syllable's stack to peak 0.5
    peak = torch.zeros(n_syl, dtype=torch.float32, device=device)
    for s0 in range(0, total, chunk):
        s1 = min(total, s0 + chunk)
        n = torch.arange(s0, s1, device=device, dtype=torch.int64)
        sid = torch.searchsorted(starts_t, n, right=True) - 1
        peak.scatter_reduce_(0, sid, torch.abs(stack[s0:s1]), reduce="amax")
    scale = 0.5 / torch.clamp(peak, min=1e-12)
    for s0 in range(0, total, chunk):
        s1 = min(total, s0 + chunk)
        n = torch.arange(s0, s1, device=device, dtype=torch.int64)
        sid = torch.searchsorted(starts_t, n, right=True) - 1
        tau = (n - starts_t[sid]).double()
        env = torch.sin(math.pi * tau / lens_t[sid].double()) ** 2
        noise = torch.randn(s1 - s0, generator=g, device=device, dtype=torch.float32) * 0.02
        out[s0:s1] = (stack[s0:s1].double() * scale[sid].double() * env).float() + noise
    return out


# ---------------------------------------------------------------------------
# Config 5 layout: per sequence, k ~ U{4..16} audio clips holding exactly
# ``audio_frames`` frames in total (each clip >= 20 frames, multinomial
# split) and k+1 text runs (each >= 1 position) filling the rest, in the
# order text, audio, text, ..., text.
# ---------------------------------------------------------------------------
def interleave_layout(seed: int = 4, n_seq: int = 256, seq_len: int = 32768,
                      audio_frac: float = 0.40, vocab: int = 131072, min_clip: int = 20):
    """Returns a dict with per-segment arrays (numpy):

    ``seg_seq, seg_kind (0 text, 1 audio), seg_start (position in its sequence),
    seg_len (positions)``, text ``ids`` for every position (ignored at audio
    positions), and ``audio_frames`` per sequence.
    """
    rng = np.random.default_rng(seed)
    audio_frames = int(round(audio_frac * seq_len))
    if audio_frac == 0.40 and seq_len == 32768:
        audio_frames = 13107
    text_pos = seq_len - audio_frames
    seg_seq, seg_kind, seg_start, seg_len = [], [], [], []
    for s in range(n_seq):
        k = int(rng.integers(4, 17))
        k = max(1, min(k, audio_frames // min_clip)) if audio_frames > 0 else 0
        if k > 0:
            extra = rng.multinomial(audio_frames - k * min_clip, np.full(k, 1.0 / k))
            clips = (extra + min_clip).tolist()
        else:
            clips = []
        n_runs = k + 1
        n_runs = min(n_runs, max(1, text_pos)) if text_pos > 0 else 0
        if n_runs > 0:
            extra = rng.multinomial(text_pos - n_runs, np.full(n_runs, 1.0 / n_runs))
            runs = (extra + 1).tolist()
        else:
            runs = []
        p = 0
        for i in range(max(len(runs), len(clips))):
            if i < len(runs):
                seg_seq.append(s); seg_kind.append(0); seg_start.append(p); seg_len.append(runs[i]); p += runs[i]
            if i < len(clips):
                seg_seq.append(s); seg_kind.append(1); seg_start.append(p); seg_len.append(clips[i]); p += clips[i]
        assert p == seq_len
    ids = rng.integers(0, vocab, size=(n_seq, seq_len), dtype=np.int64).astype(np.int32)
    return {
        "n_seq": n_seq, "seq_len": seq_len, "audio_frames": audio_frames,
        "seg_seq": np.array(seg_seq, dtype=np.int64), "seg_kind": np.array(seg_kind, dtype=np.int64),
        "seg_start": np.array(seg_start, dtype=np.int64), "seg_len": np.array(seg_len, dtype=np.int64),
        "ids": ids,
    }


def streaming_hops(seed: int = 3, n_streams: int = 4096, n_steps: int = 1000, device="cpu") -> torch.Tensor:
    """[n_steps, n_streams, 800] fp32: the hop each stream delivers at each step
    (the bursts model, 50 s per stream at the default sizes), step-major so that
    one step's hops are contiguous."""
    total = n_steps * HOP
    out = torch.empty((n_steps, n_streams, HOP), dtype=torch.float32, device=device)
    chunk = max(1, int(2 ** 26 // max(1, total)))
    for s0 in range(0, n_streams, chunk):
        s1 = min(n_streams, s0 + chunk)
        x = bursts_clips(seed * 1_000_003 + s0, s1 - s0, total, device=device)
        out[:, s0:s1, :] = x.view(s1 - s0, n_steps, HOP).permute(1, 0, 2)
    return out


# ---------------------------------------------------------------------------
# Decoder short convolution: bf16 activations ~ N(0, std) (the residual-branch
# and key / value projection outputs it is applied to), weights ~ U(-0.5, 0.5)
# per channel and tap, and ragged request lengths.
# ---------------------------------------------------------------------------
def activations_bf16(seed: int, n_tokens: int, channels: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """[n_tokens, channels] bf16 bit patterns in an int16 tensor."""
    return table_bf16(seed, rows=n_tokens, d_model=channels, std=std, device=device)


def shortconv_weight(seed: int, channels: int, width: int = 4) -> torch.Tensor:
    """[channels, width] fp32 taps ~ U(-0.5, 0.5)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.uniform(-0.5, 0.5, (channels, width)).astype(np.float32))


def request_lengths(seed: int, n: int, lo: int = 0, hi: int = 200) -> list:
    """n request lengths ~ U{lo..hi} (empty requests included when lo = 0)."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.integers(lo, hi + 1, n)]
