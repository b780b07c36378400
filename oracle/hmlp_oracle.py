"""Plain CPU oracle for the hMLP image front end (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no
code with the HIP library.

Sources:
* "Inside Inkling: Audio Design", Part 1, "Why this is a reasonable bet":
  vision uses a 4-layer hMLP over 40x40 patches.
* "Why Thinking Machines Built Inkling Without a Vision Encoder": each image
  splits into 40 x 40 pixel tiles, and every tile goes through a compact
  four-stage hMLP stem before joining the token stream.
* The architecture summary page ("simple modules rather than separate
  encoders"): a hierarchical MLP patchifier whose linear layers progressively
  merge pixels into one embedding per patch.

Readings (the pages give no widths, activation, norm or merge pattern):
* the four stages merge 5 x 5 pixels, then 2 x 2, 2 x 2 and 2 x 2 neighbours
  (40 = 5 * 2 * 2 * 2): stage 1 is a linear map of each 5 x 5 x 3 sub-patch
  flattened as (row, column, channel); stage k > 1 is a linear map of the
  2 x 2 neighbouring stage-(k-1) outputs concatenated in (row, column) order;
* widths d/4, d/4, d/4, d (d = 6144: 1536, 1536, 1536, 6144), the pattern of
  the hMLP stem the pages' source cites;
* every stage has a bias; stages 1-3 are followed by the exact GELU,
  x * Phi(x); the stem's normalisation is an inference-time affine map folded
  into the weights and biases, so it is not a separate step;
* images are bf16, height-width-channel (RGB) layout; weights bf16 [out, in],
  biases fp32; the hidden activations are stored as bf16 (round to nearest
  even) between stages; patches are numbered image by image, row-major over
  the patch grid.
The oracle evaluates each stage in fp64 and rounds the hidden activations to
bf16 at the same points.
"""

from __future__ import annotations

import numpy as np
from scipy.special import erf

PATCH = 40
FIRST = 5            # stage 1 merges 5 x 5 pixels
MERGE = 2            # stages 2..4 merge 2 x 2 neighbours
STAGES = 4
CHANNELS = 3


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_value(x) -> np.ndarray:
    """Round fp64 values to the nearest-even bf16 value (returned as fp64)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = x.view(np.uint64)
    r = (u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def gelu(x) -> np.ndarray:
    """Exact GELU, x * Phi(x) with Phi the standard normal CDF."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def num_patches(n_images: int, height: int, width: int) -> int:
    if height % PATCH or width % PATCH:
        raise ValueError("image sides must be multiples of 40")
    return n_images * (height // PATCH) * (width // PATCH)


def subpatches(images: np.ndarray) -> np.ndarray:
    """[n, H, W, 3] -> [n, H/5, W/5, 75]: each 5 x 5 x 3 block flattened (row, column, channel)."""
    n, H, W, C = images.shape
    x = images.reshape(n, H // FIRST, FIRST, W // FIRST, FIRST, C)
    return x.transpose(0, 1, 3, 2, 4, 5).reshape(n, H // FIRST, W // FIRST, FIRST * FIRST * C)


def merge2x2(h: np.ndarray) -> np.ndarray:
    """[n, h, w, C] -> [n, h/2, w/2, 4C]: the 2 x 2 neighbours concatenated in (row, column) order."""
    n, hh, ww, C = h.shape
    x = h.reshape(n, hh // 2, 2, ww // 2, 2, C)
    return x.transpose(0, 1, 3, 2, 4, 5).reshape(n, hh // 2, ww // 2, 4 * C)


def stage(x: np.ndarray, w_bits, bias, activation: bool) -> np.ndarray:
    """One stage on rows x [..., K] (fp64): x W^T + b, then GELU if activation (exact, fp64)."""
    w = bf16_bits_to_f64(w_bits)
    y = x @ w.T + np.asarray(bias, dtype=np.float64)
    return gelu(y) if activation else y


def hmlp(image_bits, weights, linear: bool = False, keep: bool = False):
    """Patch embeddings of bf16 images [n, H, W, 3] (bit patterns).

    weights: four (w_bits [out, in], bias [out]) pairs.  Returns the fp64
    embeddings [n * H/40 * W/40, d] before the final rounding (and, with
    keep=True, the list of stage inputs and outputs).  linear=True drops the
    GELU and the bf16 rounding of the hidden activations (a layout check)."""
    x = bf16_bits_to_f64(image_bits)
    if x.ndim != 4 or x.shape[3] != CHANNELS:
        raise ValueError("images must be [n, H, W, 3]")
    n, H, W, _ = x.shape
    num_patches(n, H, W)
    if len(weights) != STAGES:
        raise ValueError("four stages")
    h = subpatches(x)
    trace = []
    for k, (w, b) in enumerate(weights):
        if k > 0:
            h = merge2x2(h)
        last = k == STAGES - 1
        inp = h
        h = stage(h, w, b, activation=not last and not linear)
        if not last and not linear:
            h = f64_to_bf16_value(h)
        trace.append((inp, h))
    out = h.reshape(n * (H // PATCH) * (W // PATCH), -1)
    return (out, trace) if keep else out
