"""GPU parity of the configurable front end (the config keys n_mel_bins,
mel_vocab_size, dmel_min_value, dmel_max_value) and of the embedding in other
table layouts, through the C ABI, against the oracle on the same seeded
inputs.  Bars as in the released configuration: log-mel within 1e-3 on the
clamped value, levels exact outside a 1e-3 band around the configuration's
edges (and exact against the oracle's quantizer on the GPU's own fp32 value),
embeddings bit-exact given the same levels, RMSNorm within 1e-5 relative."""

import numpy as np
import pytest
import torch

from oracle import dmel_oracle as o
from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu

SERVING = o.Config(80, 16, -1.5, 2.0)   # the serving code's default clamp minimum
CONFIGS = [
    ("serving_min_-1.5", SERVING),
    ("40x8_[-5,1]", o.Config(40, 8, -5.0, 1.0)),
    ("64x16", o.Config(64, 16, -7.0, 2.0)),
    ("37x10_[-7,2]", o.Config(37, 10, -7.0, 2.0)),
    ("80x1", o.Config(80, 1, -7.0, 2.0)),
    ("1x16", o.Config(1, 16, -7.0, 2.0)),
    ("128x32_frontend_only", o.Config(128, 32, -7.0, 2.0)),
    ("80x256_frontend_only", o.Config(80, 256, -10.0, 3.0)),
]


@pytest.fixture(scope="module")
def dm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from encoder_free_audio_amd import dmel
    return dmel


@pytest.fixture(scope="module")
def P():
    from tests import _parity
    return _parity


@pytest.fixture(scope="module")
def audio():
    # ragged clips of the pink-noise + burst model: 3 s, 2.01 s, 0.5 s, 4 s
    lengths = [48000, 32160, 8000, 64000]
    x = synth.bursts_clips(seed=11, n_clips=4, n_samples=64000).numpy()
    clips = [x[c, :n] for c, n in enumerate(lengths)]
    return lengths, clips


def _cfg_dict(c):
    return dict(n_mel_bins=c.n_mel_bins, mel_vocab_size=c.mel_vocab_size, min_value=c.min_value,
                max_value=c.max_value)


@pytest.mark.parametrize("name,cfg", CONFIGS, ids=[n for n, _ in CONFIGS])
def test_config_frontend_and_forward(dm, P, audio, name, cfg):
    lengths, clips = audio
    print(f"case: config {name}, seed 11, clips {lengths}", flush=True)
    ctx = dm.dmel_create_config(0, _cfg_dict(cfg))
    try:
        assert dm.dmel_get_config(ctx) == _cfg_dict(cfg)
        flat = P.to_dev(np.concatenate(clips))
        lm, lv = P.gpu_frames(ctx, flat, lengths, n_mels=cfg.n_mel_bins)
        ora = [o.levels_cfg(c, cfg) for c in clips]
        ora_lm = np.concatenate([a for a, _ in ora])
        ora_lv = np.concatenate([b for _, b in ora])
        assert lm.shape == ora_lm.shape == (sum(n // 800 for n in lengths), cfg.n_mel_bins)
        P.check_logmel(lm, ora_lm, cfg.min_value, cfg.max_value)
        band, forgiven, frames = P.check_levels(lv, ora_lm, ora_lv, gpu_lm=lm, cfg=cfg)
        print(f"edge band {band}, forgiven {forgiven} in {frames} frames")
        T = lm.shape[0]
        d = 256
        table = synth.table_bf16(seed=77, rows=cfg.n_mel_bins * cfg.mel_vocab_size, d_model=d)
        so, fo, _ = P.offsets(lengths)
        out = torch.empty((T, d), dtype=torch.int16, device="cuda")
        ws = torch.empty(dm.dmel_forward_workspace_bytes(T), dtype=torch.uint8, device="cuda")
        args = (ctx, flat, flat.numel(), so, fo, len(lengths), T, None, table.cuda(), d, None, None, 1e-6, out,
                dm.DMEL_BF16, d, None, ws, ws.numel())
        if cfg.n_mel_bins > 80 or cfg.mel_vocab_size > 16:
            # outside the embedding's layouts: rejected before any launch
            with pytest.raises(dm.DmelError) as e:
                dm.dmel_forward(*args)
            assert e.value.code == -2
            return
        dm.dmel_forward(*args)
        torch.cuda.synchronize()
        # the forward's levels are the standalone levels
        assert np.array_equal(ws[: T * cfg.n_mel_bins].view(T, cfg.n_mel_bins).cpu().numpy(), lv)
        got = out.cpu().numpy().view(np.uint16)
        tb = table.numpy().view(np.uint16)
        want, _ = o.embed(lv, tb, n_levels=cfg.mel_vocab_size)
        assert np.array_equal(got, want)
    finally:
        torch.cuda.synchronize()
        dm.dmel_destroy(ctx)


def test_serving_clamp_changes_only_the_quantizer(dm, P, audio):
    lengths, clips = audio
    print("case: released vs serving clamp minimum, seed 11", flush=True)
    c0 = dm.dmel_create(0)
    c1 = dm.dmel_create_config(0, _cfg_dict(SERVING))
    try:
        flat = P.to_dev(np.concatenate(clips))
        lm0, lv0 = P.gpu_frames(c0, flat, lengths)
        lm1, lv1 = P.gpu_frames(c1, flat, lengths)
        # same filterbank: bit-identical log-mel; levels differ where the
        # log-mel lies between -7 and -1.5 or crosses other edges
        assert np.array_equal(lm0.view(np.uint32), lm1.view(np.uint32))
        assert np.array_equal(lv1, o.quantize(lm1.astype(np.float64), -1.5, 2.0, 16))
        assert np.array_equal(lv0, o.quantize(lm0.astype(np.float64)))
        assert not np.array_equal(lv0, lv1)
        assert np.all(lv1[lm1 <= -1.5] == 0)
    finally:
        torch.cuda.synchronize()
        dm.dmel_destroy(c0)
        dm.dmel_destroy(c1)


LAYOUTS = [(40, 8), (64, 16), (37, 10), (41, 16), (80, 8), (80, 1), (1, 16), (2, 3), (79, 15)]


@pytest.mark.parametrize("n_bins,n_levels", LAYOUTS)
def test_embed_layouts_bit_exact(dm, P, n_bins, n_levels):
    rng = np.random.default_rng(1000 + 17 * n_bins + n_levels)
    for n, d in ((2 * 1024 + 37, 64), (5, 6144)):
        print(f"case: layout {n_bins} x {n_levels}, n={n}, d_model={d}", flush=True)
        t = synth.table_bf16(seed=200 + n_bins, rows=n_bins * n_levels, d_model=d)
        lv = rng.integers(0, n_levels, size=(n, n_bins)).astype(np.uint8)
        tb = t.numpy().view(np.uint16)
        for dt in ("f32", "bf16"):
            got = P.gpu_embed(lv, t, d, out_dtype=dt, n_levels=n_levels)
            want, _ = o.embed(lv, tb, out_dtype=dt, n_levels=n_levels)
            if dt == "f32":
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
            else:
                assert np.array_equal(got, want)
        # RMSNorm through the Gram matrix of this layout
        w = rng.uniform(0.5, 1.5, d).astype(np.float32)
        got32 = P.gpu_embed(lv, t, d, out_dtype="f32", rms_weight=w, n_levels=n_levels)
        _, exact = o.embed(lv, tb, rms_weight=w, n_levels=n_levels)
        P.check_rms_f32(got32, exact)


def test_embed_layout_clamps_levels_and_reads_unaligned(dm, P):
    # levels >= n_levels read as n_levels - 1; a non-released layout takes any
    # byte alignment of the levels array
    n_bins, n_levels, d, n = 40, 8, 128, 700
    rng = np.random.default_rng(8)
    t = synth.integer_table(seed=9, rows=n_bins * n_levels, d_model=d)
    tab = o.bf16_to_f32(t.numpy().view(np.uint16)).astype(np.int64)
    lv = rng.integers(0, 256, size=(n, n_bins)).astype(np.uint8)
    buf = torch.zeros(n * n_bins + 16, dtype=torch.uint8, device="cuda")
    buf[3: 3 + n * n_bins] = torch.from_numpy(lv.reshape(-1)).cuda()
    out = torch.empty((n, d), dtype=torch.float32, device="cuda")
    dm.dmel_embed(buf[3:], n, t.cuda(), d, None, None, out, dm.DMEL_F32, d, n_bins=n_bins, n_levels=n_levels)
    torch.cuda.synchronize()
    rows = n_levels * np.arange(n_bins)[None, :] + np.minimum(lv, n_levels - 1).astype(np.int64)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), tab[rows].sum(axis=1))


def test_layout_scale_same_for_both_kernels(dm, P):
    # batches above 131072 tokens stage G in LDS; smaller ones read it
    # directly: the scales of a token agree bit for bit in any layout
    n_bins, n_levels, d = 41, 12, 6144
    n_big = 131072 + 2049
    rng = np.random.default_rng(12)
    print("case: layout 41 x 12, scale kernels, n=133121", flush=True)
    t = synth.table_bf16(seed=13, rows=n_bins * n_levels, d_model=d).cuda()
    gram = torch.empty((1280, 1280), dtype=torch.float64, device="cuda")
    dm.dmel_rms_gram(t, d, gram, n_bins=n_bins, n_levels=n_levels)
    lv = torch.from_numpy(rng.integers(0, n_levels, size=(n_big, n_bins)).astype(np.uint8)).cuda()
    big = torch.empty(n_big, dtype=torch.float32, device="cuda")
    dm.dmel_rms_scale(lv, n_big, gram, d, 1e-6, big, n_bins=n_bins, n_levels=n_levels)
    small = torch.empty(4096, dtype=torch.float32, device="cuda")
    dm.dmel_rms_scale(lv[:4096], 4096, gram, d, 1e-6, small, n_bins=n_bins, n_levels=n_levels)
    torch.cuda.synchronize()
    assert torch.equal(big[:4096], small)
    # the Gram matrix: zero outside the layout, E E^T inside it
    g = gram.cpu().numpy().astype(np.float64)
    r = 16 * np.arange(80)[:, None] + np.arange(16)[None, :]
    inside = (np.arange(80)[:, None] < n_bins) & (np.arange(16)[None, :] < n_levels)
    assert np.all(g[~inside.reshape(-1)] == 0) and np.all(g[:, ~inside.reshape(-1)] == 0)
    e = o.bf16_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)
    idx = r[inside]
    sub = g[np.ix_(idx[:50], idx[:50])]
    src = (n_levels * (idx[:50] // 16) + idx[:50] % 16)
    ref = e[src] @ e[src].T
    assert np.max(np.abs(sub - ref) / np.maximum(np.abs(ref), 1e-3)) < 1e-11
    # and the sampled scales against the oracle's norm
    lvn = lv[:64].cpu().numpy()
    s = o.embed_sum(lvn, t.cpu().numpy().view(np.uint16), n_levels=n_levels).astype(np.float64)
    want = 1.0 / np.sqrt(np.mean(s * s, axis=1) + 1e-6)
    assert np.max(np.abs(small[:64].cpu().numpy() / want - 1.0)) < 1e-5
