"""Plain CPU oracle for the decoder's short convolution (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no
code with the HIP library.

Source: "Inside Inkling: Audio Design", Part 3 - Inference, the bullet on
short convolutions: per-channel causal convolutions of width W = 4,
y[t, c] = x[t, c] + sum_{d=0}^{W-1} w[c, d] * x[t - d, c]; and the subsection
"Where audio touches the serving path": the branch keeps a small
per-request convolution state.

Readings where the page is silent:
* the state of a request is its last W - 1 = 3 inputs, oldest first; the
  inputs before a request's first token are that state (zeros for a new
  request), and after a chunk the state is the last 3 inputs of the
  concatenation [state, chunk] (so a chunk shorter than 3 keeps part of the
  old state);
* x and the state are bf16 (the decoder's activation type), the weights fp32;
  the oracle evaluates the formula exactly in fp64 (every bf16 and fp32 input
  is exact in fp64, and the five-term sum is then rounded once).
"""

from __future__ import annotations

import numpy as np

WIDTH = 4
STATE = WIDTH - 1


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def shortconv(x_bits, seq_off, weight, state_bits=None):
    """Short convolution of ragged requests.

    x_bits     uint16 [T, C] bf16 bit patterns; request s is rows
               seq_off[s] .. seq_off[s+1]
    weight     [C, 4] (w[c, d] multiplies x[t - d, c])
    state_bits uint16 [S, 3, C] or None (zeros): x[-3], x[-2], x[-1] of each request
    Returns (y fp64 [T, C], state_out uint16 [S, 3, C]).
    """
    x = bf16_bits_to_f64(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be [T, C]")
    T, C = x.shape
    off = np.asarray(seq_off, dtype=np.int64)
    S = off.size - 1
    if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("bad sequence offsets")
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (C, WIDTH):
        raise ValueError("weight must be [C, 4]")
    if state_bits is None:
        state_bits = np.zeros((S, STATE, C), dtype=np.uint16)
    state_bits = np.asarray(state_bits, dtype=np.uint16)
    y = np.empty((T, C), dtype=np.float64)
    state_out = np.empty((S, STATE, C), dtype=np.uint16)
    x_in = np.asarray(x_bits, dtype=np.uint16)
    for s in range(S):
        a, b = int(off[s]), int(off[s + 1])
        xp = np.concatenate([bf16_bits_to_f64(state_bits[s]), x[a:b]], axis=0)   # [3 + n, C]
        n = b - a
        for t in range(n):
            k = STATE + t       # row of x[t] in xp
            acc = xp[k].copy()
            for d in range(WIDTH):
                acc += w[:, d] * xp[k - d]
            y[a + t] = acc
        tail = np.concatenate([state_bits[s], x_in[a:b]], axis=0)
        state_out[s] = tail[-STATE:]
    return y, state_out
