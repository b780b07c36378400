"""The allocation-free forward (dmel_forward_noalloc) against dmel_forward
with a workspace: the same kernels, so the same bits.  Two calls in a row on
the library's scratch, the second with a smaller batch (its contents are the
first call's leftovers, which must not matter), plus the size limit."""

import numpy as np
import pytest
import torch

from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from encoder_free_audio_amd import dmel as dm
    ctx = dm.dmel_create(0)
    table = synth.table_bf16(1234).cuda()
    gram = torch.empty((1280, 1280), dtype=torch.float64, device="cuda")
    dm.dmel_rms_gram(table, 6144, gram)
    w = (torch.rand(6144, generator=torch.Generator().manual_seed(9)) + 0.5).cuda()
    yield dm, ctx, table, gram, w
    torch.cuda.synchronize()
    dm.dmel_destroy(ctx)


def _both(dm, ctx, table, gram, w, audio, lengths, rms, out_dtype):
    so, fo, T = dm.clip_offsets(lengths, "cuda")
    n = audio.numel()
    tdt = torch.int16 if out_dtype == dm.DMEL_BF16 else torch.float32
    ref = torch.empty((T, 6144), dtype=tdt, device="cuda")
    got = torch.full((T, 6144), 7, dtype=tdt, device="cuda")
    ws = torch.empty(dm.dmel_forward_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    wgt, g = (w, gram) if rms else (None, None)
    dm.dmel_forward(ctx, audio, n, so, fo, len(lengths), T, None, table, 6144, wgt, g, 1e-6, ref, out_dtype, 6144,
                    None, ws, ws.numel())
    dm.dmel_forward_noalloc(ctx, audio, n, so, fo, len(lengths), T, None, table, 6144, wgt, g, 1e-6, got, out_dtype,
                            6144, None)
    torch.cuda.synchronize()
    return ref, got, T


@pytest.mark.parametrize("rms", [True, False])
def test_noalloc_equals_forward_two_calls(env, rms):
    dm, ctx, table, gram, w = env
    out_dtype = dm.DMEL_BF16 if rms else dm.DMEL_F32
    # first call: 8 x 30 s (4800 frames), then 3 ragged clips (455 frames)
    big = synth.bursts_clips(seed=1, n_clips=8, n_samples=480000).cuda().reshape(-1)
    print(f"case: noalloc, rms={rms}, 4800 frames then 455", flush=True)
    ref, got, T = _both(dm, ctx, table, gram, w, big, [480000] * 8, rms, out_dtype)
    assert T == 4800 and torch.equal(ref, got)
    lengths = [160000, 123456, 80800]
    small = synth.speech_clips(seed=6, lengths=lengths, device="cuda")
    ref, got, T = _both(dm, ctx, table, gram, w, small, lengths, rms, out_dtype)
    assert T == sum(n // 800 for n in lengths) and torch.equal(ref, got)


def test_noalloc_rejects_batches_beyond_the_scratch(env):
    dm, ctx, table, gram, w = env
    T = dm.NOALLOC_MAX_FRAMES + 1
    so, fo, _ = dm.clip_offsets([T * 800], "cuda")
    dummy = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(dm.DmelError) as e:
        # validation only: fails on the frame count before any work is enqueued
        dm.dmel_forward_noalloc(ctx, dummy, T * 800, so, fo, 1, T, None, table, 6144, None, None, 1e-6, dummy,
                                dm.DMEL_F32, 6144, None)
    assert "DMEL_ENOMEM" in str(e.value)
