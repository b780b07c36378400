"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the same arrays, and compare to the stated bars.

Bars (per element):
* log-mel: |gpu - oracle| <= 1e-3 on values clamped to [-7, 2] (or the
  configuration's clamp range); where the oracle is below the minimum the
  GPU value only has to be <= minimum + 1e-3.
* levels: equal, except where the oracle's log-mel lies within 1e-3 of a
  decision edge (-7 + 9k/16 for the released quantizer) (those are
  counted); and always equal to the oracle's quantizer applied to the GPU's
  own fp32 log-mel.
* embedding without RMSNorm: bit-exact given the same levels.
* RMSNorm: fp32 output within 1e-5 relative of the oracle's fp64 value; bf16
  output equal, or one ulp apart where the oracle value is within 1e-5
  relative of a bf16 rounding midpoint.
"""

from __future__ import annotations

import numpy as np
import torch

from encoder_free_audio_amd import dmel as dm
from oracle import dmel_oracle as o

LOGMEL_TOL = 1e-3
RMS_TOL = 1e-5
DEV = "cuda"


def to_dev(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def offsets(lengths):
    return dm.clip_offsets(lengths, DEV)


def gpu_frames(ctx, audio_flat: torch.Tensor, lengths, carry=None, n_mels=80):
    """(logmel fp32 [T,n_mels], levels u8 [T,n_mels]) from the HIP path, as numpy."""
    so, fo, T = offsets(lengths)
    lm = torch.empty((max(T, 1), n_mels), dtype=torch.float32, device=DEV)
    lv = torch.empty((max(T, 1), n_mels), dtype=torch.uint8, device=DEV)
    n = audio_flat.numel()
    dm.dmel_frames(ctx, audio_flat, n, so, fo, len(lengths), T, carry, lm)
    dm.dmel_levels(ctx, audio_flat, n, so, fo, len(lengths), T, carry, lv)
    torch.cuda.synchronize()
    return lm[:T].cpu().numpy(), lv[:T].cpu().numpy()


def gpu_embed(levels_np, table_bits: torch.Tensor, d_model, out_dtype="bf16", rms_weight=None, eps=1e-6,
              gram=None, n_levels=16):
    n, n_bins = levels_np.shape
    lay = dict(n_bins=n_bins, n_levels=n_levels)
    lv = to_dev(levels_np.astype(np.uint8))
    table = table_bits.to(DEV)
    dt = dm.DMEL_BF16 if out_dtype == "bf16" else dm.DMEL_F32
    out = torch.empty((max(n, 1), d_model), dtype=torch.int16 if dt == dm.DMEL_BF16 else torch.float32,
                      device=DEV)
    w = None
    scale = None
    if rms_weight is not None:
        w = to_dev(np.asarray(rms_weight, dtype=np.float32))
        if gram is None:
            gram = torch.empty((1280, 1280), dtype=torch.float64, device=DEV)
            dm.dmel_rms_gram(table, d_model, gram, **lay)
        scale = torch.empty(max(n, 1), dtype=torch.float32, device=DEV)
        dm.dmel_rms_scale(lv, n, gram, d_model, eps, scale, **lay)
    dm.dmel_embed(lv, n, table, d_model, w, scale, out, dt, d_model, **lay)
    torch.cuda.synchronize()
    res = out[:n].cpu().numpy()
    return res.view(np.uint16) if dt == dm.DMEL_BF16 else res


def check_logmel(gpu_lm, ora_lm, lo=o.CLAMP_MIN, hi=o.CLAMP_MAX):
    g = np.asarray(gpu_lm, dtype=np.float64)
    r = np.asarray(ora_lm, dtype=np.float64)
    assert g.shape == r.shape
    gc = np.clip(g, lo, hi)
    rc = np.clip(r, lo, hi)
    err = np.abs(gc - rc)
    assert err.max(initial=0.0) <= LOGMEL_TOL, f"clamped log-mel error {err.max()}"
    below = r < lo
    if below.any():
        assert g[below].max() <= lo + LOGMEL_TOL
    above = r >= lo
    return float(err.max(initial=0.0)), float(np.abs(g - r)[above].max(initial=0.0))


def check_levels(gpu_lv, ora_lm, ora_lv, gpu_lm=None, cfg=None):
    """Returns (elements in the edge band, forgiven mismatches, frames affected).

    cfg: an oracle Config for a non-released quantizer (None: released)."""
    cfg = cfg or o.Config()
    q = (cfg.min_value, cfg.max_value, cfg.mel_vocab_size)
    gpu_lv = np.asarray(gpu_lv)
    ora_lv = np.asarray(ora_lv)
    assert gpu_lv.shape == ora_lv.shape
    assert gpu_lv.max(initial=0) <= cfg.mel_vocab_size - 1
    edges = o.level_edges(*q)
    if edges.size == 0:
        assert np.array_equal(gpu_lv, ora_lv)
        return 0, 0, 0
    d = np.min(np.abs(np.asarray(ora_lm, dtype=np.float64)[..., None] - edges), axis=-1)
    band = d <= LOGMEL_TOL
    mism = gpu_lv != ora_lv
    bad = mism & ~band
    assert not bad.any(), f"{int(bad.sum())} level mismatches outside the edge band"
    # a mismatch inside the band can only be one level apart
    assert np.all(np.abs(gpu_lv.astype(int) - ora_lv.astype(int))[mism] == 1)
    if gpu_lm is not None:
        # the same decision taken on the GPU's own fp32 value: exact
        same = o.quantize(np.asarray(gpu_lm, dtype=np.float32), *q)
        assert np.array_equal(same, gpu_lv)
    frames = int(np.any(mism, axis=-1).sum()) if mism.ndim == 2 else int(mism.any())
    return int(band.sum()), int(mism.sum()), frames


def check_rms_f32(gpu, exact):
    g = np.asarray(gpu, dtype=np.float64)
    e = np.asarray(exact, dtype=np.float64)
    rel = np.abs(g - e) / np.maximum(np.abs(e), 1e-30)
    assert rel.max(initial=0.0) <= RMS_TOL, f"RMSNorm relative error {rel.max()}"
    return float(rel.max(initial=0.0))


def check_rms_bf16(gpu_bits, exact):
    """bf16 output vs the oracle's fp64 value; returns the number of 1-ulp
    differences (all of them next to a rounding midpoint)."""
    want = o.f64_to_bf16(exact)
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    diff = gpu_bits != want
    if not diff.any():
        return 0
    e = np.asarray(exact, dtype=np.float64)[diff]
    gv = o.bf16_to_f32(gpu_bits[diff]).astype(np.float64)
    wv = o.bf16_to_f32(want[diff]).astype(np.float64)
    mid = 0.5 * (gv + wv)
    ok = np.abs(e - mid) <= RMS_TOL * np.abs(e)
    ulp = np.abs(gpu_bits[diff].astype(np.int64) - want[diff].astype(np.int64)) == 1
    assert np.all(ok & ulp), f"{int((~(ok & ulp)).sum())} bf16 RMSNorm outputs differ away from a midpoint"
    return int(diff.sum())
