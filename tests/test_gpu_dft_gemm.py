"""GPU parity of the DFT-as-GEMM front end of the benchmark-only library
(dmel_bench_frames_dft_gemm, the measured alternative to the FFT): its log-mel
against the CPU oracle, to the same bar as dmel_frames (|dl| <= 1e-3 on values
clamped to [-7, 2]; values below the clamp only need to stay below it)."""

import numpy as np
import pytest
import torch

from oracle import dmel_oracle as o
from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu

P = None


@pytest.fixture(scope="module")
def env():
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import _parity
    from encoder_free_audio_amd import bench_ext as be
    from encoder_free_audio_amd import dmel
    P = _parity
    ctx = dmel.dmel_create(0)
    mat = torch.empty(be.dmel_bench_dft_matrix_bytes(), dtype=torch.uint8, device="cuda")
    be.dmel_bench_dft_matrix(mat)
    yield be, ctx, mat
    torch.cuda.synchronize()
    dmel.dmel_destroy(ctx)


def gemm_frames(dm, ctx, mat, flat, lengths, carry=None):
    so, fo, T = P.offsets(lengths)
    lm = torch.empty((max(T, 1), 80), dtype=torch.float32, device="cuda")
    wsb = dm.dmel_bench_dft_gemm_workspace_bytes(T)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    dm.dmel_bench_frames_dft_gemm(ctx, flat, flat.numel(), so, fo, len(lengths), T, carry, mat, lm, ws, wsb)
    torch.cuda.synchronize()
    return lm[:T].cpu().numpy()


def test_dft_matrix_values(env):
    # the split matrix reproduces cos / -sin to ~2^-16 and its padding rows and bias are zero
    dm, ctx, mat = env
    nb = 1792 * 4800 * 2
    B = mat[:nb].view(torch.int16).view(torch.bfloat16).float().view(1792, 4800).cpu().numpy().astype(np.float64)
    bias = mat[nb:].view(torch.float32).cpu().numpy()
    n = np.arange(1600)
    for j in (0, 1, 2, 399, 400, 800, 801, 802, 1200, 1601):
        k = j if j < 801 else j - 801
        want = np.cos(2 * np.pi * k * n / 1600) if j < 801 else -np.sin(2 * np.pi * k * n / 1600)
        got = B[j, :1600] + B[j, 1600:3200]
        assert np.max(np.abs(got - want)) < 2.0 ** -16, j
        assert np.array_equal(B[j, :1600], B[j, 3200:])
    assert not B[1602:].any() and not bias.any()


def test_tones_and_bursts(env):
    dm, ctx, mat = env
    x = synth.tones_clip(seed=0)
    print("case: dft-gemm, 1 s of three tones", flush=True)
    lm = gemm_frames(dm, ctx, mat, P.to_dev(x), [x.size])
    err, _ = P.check_logmel(lm, o.log_mel(x))
    print(f"tones: max |dl| {err:.2e}")
    xb = synth.bursts_clips(seed=1, n_clips=8, n_samples=480000).numpy()
    print("case: dft-gemm, 8 x 30 s bursts", flush=True)
    lm = gemm_frames(dm, ctx, mat, P.to_dev(xb.reshape(-1)), [480000] * 8)
    ora = np.concatenate([o.log_mel(xb[c]) for c in range(8)])
    err, _ = P.check_logmel(lm, ora)
    print(f"bursts: max |dl| {err:.2e}")


def test_speech_and_ragged_carry(env):
    dm, ctx, mat = env
    xs = synth.speech_clips(2, [16000 * 12, 16000 * 7 + 123]).numpy()
    lengths = [16000 * 12, 16000 * 7 + 123]
    print("case: dft-gemm, speech-like clips", flush=True)
    lm = gemm_frames(dm, ctx, mat, P.to_dev(xs), lengths)
    ora = np.concatenate([o.log_mel(xs[:lengths[0]]), o.log_mel(xs[lengths[0]:])])
    err, _ = P.check_logmel(lm, ora)
    print(f"speech: max |dl| {err:.2e}")
    rng = np.random.default_rng(31)
    lengths = [0, 799, 800, 1601, 16123, 2400, 0, 8000]
    clips = [(rng.standard_normal(n) * 0.1).astype(np.float32) for n in lengths]
    flat = np.concatenate(clips)
    carry = (rng.standard_normal((len(lengths), 800)) * 0.1).astype(np.float32)
    for use_carry in (False, True):
        print(f"case: dft-gemm, ragged clips {lengths} carry={use_carry}", flush=True)
        lm = gemm_frames(dm, ctx, mat, P.to_dev(flat), lengths, carry=P.to_dev(carry) if use_carry else None)
        ora = np.concatenate([o.log_mel(clips[c], carry[c] if use_carry else None) for c in range(len(lengths))])
        assert lm.shape == ora.shape
        P.check_logmel(lm, ora)
