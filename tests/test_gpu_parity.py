"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs (sizes the oracle finishes in seconds; several
workgroup tiles and ragged tails)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import dmel_oracle as o
from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu

P = None  # tests/_parity.py, imported lazily (it needs torch.cuda)


@pytest.fixture(scope="module")
def env():
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import _parity
    from encoder_free_audio_amd import dmel as dm
    P = _parity
    ctx = dm.dmel_create(0)
    yield dm, ctx
    torch.cuda.synchronize()
    dm.dmel_destroy(ctx)


@pytest.fixture(scope="module")
def table():
    return synth.table_bf16(1234)


def _tbits(t):
    return t.numpy().view(np.uint16)


# ---------------------------------------------------------------------------
def test_c1_tones_end_to_end(env, table):
    dm, ctx = env
    x = synth.tones_clip(seed=0)
    print("case: 1 s of three tones, seed 0", flush=True)
    lm, lv = P.gpu_frames(ctx, P.to_dev(x), [x.size])
    ora_lm = o.log_mel(x)
    ora_lv = o.quantize(ora_lm)
    assert lm.shape == (20, 80)
    P.check_logmel(lm, ora_lm)
    band, forgiven, frames = P.check_levels(lv, ora_lm, ora_lv, gpu_lm=lm)
    print(f"edge band {band}, forgiven {forgiven} in {frames} frames")
    # the first 0.25 s is exact silence: frames 0..4 are all level 0
    assert np.all(lv[:5] == 0) and np.max(np.abs(lm[:5] - np.log(1e-10))) < 1e-5
    tb = _tbits(table)
    for dt in ("bf16", "f32"):
        got = P.gpu_embed(ora_lv, table, 6144, out_dtype=dt)
        want, _ = o.embed(ora_lv, tb, out_dtype=dt)
        assert np.array_equal(got.view(np.uint32) if dt == "f32" else got,
                              want.view(np.uint32) if dt == "f32" else want)
    # end to end through dmel_forward
    so, fo, T = P.offsets([x.size])
    out = torch.empty((T, 6144), dtype=torch.int16, device="cuda")
    ws = torch.empty(dm.dmel_forward_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    dm.dmel_forward(ctx, P.to_dev(x), x.size, so, fo, 1, T, None, table.cuda(), 6144, None, None, 1e-6,
                    out, dm.DMEL_BF16, 6144, None, ws, ws.numel())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want, _ = o.embed(ora_lv, tb)
    same = np.all(lv == ora_lv, axis=1)
    assert same.sum() >= T - frames
    assert np.array_equal(got[same], want[same])


def test_c2_bursts_rmsnorm(env, table):
    dm, ctx = env
    x = synth.bursts_clips(seed=1, n_clips=8, n_samples=480000).numpy()
    print("case: 8 x 30 s pink noise + bursts, seed 1", flush=True)
    flat = x.reshape(-1)
    lm, lv = P.gpu_frames(ctx, P.to_dev(flat), [480000] * 8)
    assert lm.shape == (4800, 80)
    ora_lm = np.concatenate([o.log_mel(x[c]) for c in range(8)])
    ora_lv = o.quantize(ora_lm)
    err, _ = P.check_logmel(lm, ora_lm)
    band, forgiven, frames = P.check_levels(lv, ora_lm, ora_lv, gpu_lm=lm)
    print(f"log-mel max err {err:.2e}; edge band {band} ({band / lv.size:.4%}), forgiven {forgiven} in {frames} frames")
    # at least 10% of the samples are silent: whole silent frames give level 0
    assert (lv == 0).all(axis=1).sum() > 0
    # RMSNorm (w = 1, eps 1e-6) on clips 0 and 7, fed the oracle's levels
    tb = _tbits(table)
    sel = np.r_[0:600, 4200:4800]
    w = np.ones(6144, dtype=np.float32)
    got32 = P.gpu_embed(ora_lv[sel], table, 6144, out_dtype="f32", rms_weight=w)
    _, exact = o.embed(ora_lv[sel], tb, rms_weight=w)
    rel = P.check_rms_f32(got32, exact)
    got16 = P.gpu_embed(ora_lv[sel], table, 6144, out_dtype="bf16", rms_weight=w)
    nd = P.check_rms_bf16(got16, exact)
    print(f"RMSNorm max rel err {rel:.2e}; bf16 midpoint differences {nd}")


def test_rmsnorm_weight_released_layout(env, table):
    # a non-unit RMSNorm weight on the released 80 x 16 layout, fp32 and bf16
    # out, against the oracle: the levels of the 8 x 30 s bursts workload
    dm, ctx = env
    x = synth.bursts_clips(seed=1, n_clips=8, n_samples=480000).numpy()
    print("case: 8 x 30 s bursts, RMSNorm weight U(0.5, 1.5)", flush=True)
    ora_lv = np.concatenate([o.levels(x[c]) for c in range(8)])
    w = np.random.default_rng(31).uniform(0.5, 1.5, 6144).astype(np.float32)
    tb = _tbits(table)
    _, exact = o.embed(ora_lv, tb, rms_weight=w)
    rel = P.check_rms_f32(P.gpu_embed(ora_lv, table, 6144, out_dtype="f32", rms_weight=w), exact)
    nd = P.check_rms_bf16(P.gpu_embed(ora_lv, table, 6144, out_dtype="bf16", rms_weight=w), exact)
    _record_rms("rmsnorm_weight_bursts", rel, nd, ora_lv.shape[0])


def _cancelling_table(sigma, seed=5):
    # rows of bin j = (-1)^j mu + N(0, sigma): the 80 rows a token selects
    # cancel, so |s|^2 is far smaller than the sum of the Gram terms
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal(6144)
    mu *= np.sqrt(10.0) / np.linalg.norm(mu)
    sign = np.where(np.arange(80) % 2 == 0, 1.0, -1.0)
    e = np.repeat(sign, 16)[:, None] * mu[None, :] + sigma * rng.standard_normal((1280, 6144))
    return torch.from_numpy(o.f32_to_bf16(e.astype(np.float32)).view(np.int16).copy())


@pytest.mark.parametrize("sigma", [0.02, 0.002])
def test_rmsnorm_cancelling_table(env, sigma):
    dm, ctx = env
    print(f"case: cancelling table |mu|^2 = 10, sigma {sigma}, random weight", flush=True)
    t = _cancelling_table(sigma)
    rng = np.random.default_rng(32)
    lv = rng.integers(0, 16, (2 * 1024 + 37, 80)).astype(np.uint8)
    w = rng.uniform(0.5, 1.5, 6144).astype(np.float32)
    _, exact = o.embed(lv, _tbits(t), rms_weight=w)
    rel = P.check_rms_f32(P.gpu_embed(lv, t, 6144, out_dtype="f32", rms_weight=w), exact)
    nd = P.check_rms_bf16(P.gpu_embed(lv, t, 6144, out_dtype="bf16", rms_weight=w), exact)
    _record_rms(f"rmsnorm_cancelling_sigma{sigma}", rel, nd, lv.shape[0])


def _record_rms(case, rel, nd, n):
    from tests import _record
    _record.record(case, tokens=int(n), max_rel_err_f32=rel, bf16_midpoint_ulps=nd)
    print(f"{case}: max rel err {rel:.2e}; bf16 midpoint differences {nd}")


def test_embed_tiles_and_ragged_tail(env):
    dm, ctx = env
    rng = np.random.default_rng(21)
    for n, d in ((2 * 1024 + 37, 256), (1, 16), (300, 6144), (1024, 48)):
        print(f"case: random levels n={n} d_model={d}", flush=True)
        t = synth.table_bf16(seed=100 + d, d_model=d)
        lv = rng.integers(0, 16, size=(n, 80)).astype(np.uint8)
        tb = _tbits(t)
        got = P.gpu_embed(lv, t, d, out_dtype="f32")
        want, _ = o.embed(lv, tb, out_dtype="f32")
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        got = P.gpu_embed(lv, t, d, out_dtype="bf16")
        want, _ = o.embed(lv, tb)
        assert np.array_equal(got, want)


def test_embed_fixed_order_golden(env, golden_dir):
    dm, ctx = env
    with open(os.path.join(golden_dir, "fixed_order.json")) as f:
        c = json.load(f)
    d = 16
    table = np.full((1280, d), np.float32(c["poison"]), dtype=np.float32)
    L = np.array([(7 * j + 3) % 16 for j in range(80)])
    r = 16 * np.arange(80) + L
    col = np.zeros((80, 5), dtype=np.float64)
    col[:, 0] = 2.0 ** -24
    col[0, 0] = 1.0
    col[0, 1], col[1, 1], col[2, 1] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    col[0, 2], col[1, 2] = 1.0, 1.5 * 2.0 ** -24
    col[:, 3] = np.arange(80)
    col[:, 4] = -0.0
    table[r, :5] = col.astype(np.float32)
    bits = o.f32_to_bf16(table)
    t = torch.from_numpy(bits.view(np.int16).copy())
    got = P.gpu_embed(L[None, :].astype(np.uint8), t, d, out_dtype="f32")[0]
    want = np.array([int(x["expect_f32_hex"], 16) for x in c["columns"]], dtype=np.uint32)
    assert np.array_equal(got[:5].view(np.uint32), want)
    got16 = P.gpu_embed(L[None, :].astype(np.uint8), t, d, out_dtype="bf16")[0]
    want16 = np.array([int(x["expect_bf16_hex"], 16) for x in c["columns"]], dtype=np.uint16)
    assert np.array_equal(got16[:5], want16)


def test_integer_table_and_level_clamp(env):
    dm, ctx = env
    t = synth.integer_table(seed=5, d_model=64)
    tab = o.bf16_to_f32(_tbits(t)).astype(np.int64)
    rng = np.random.default_rng(6)
    lv = rng.integers(0, 256, size=(50, 80)).astype(np.uint8)   # values > 15 read as 15
    got = P.gpu_embed(lv, t, 64, out_dtype="f32")
    lvc = np.minimum(lv, 15).astype(np.int64)
    rows = 16 * np.arange(80)[None, :] + lvc
    want = tab[rows].sum(axis=1)
    assert np.array_equal(got.astype(np.int64), want)


def test_ragged_clips_with_carry(env, table):
    dm, ctx = env
    rng = np.random.default_rng(31)
    lengths = [0, 799, 800, 1601, 16123, 2400, 0, 8000]
    clips = [(rng.standard_normal(n) * 0.1).astype(np.float32) for n in lengths]
    flat = np.concatenate(clips) if sum(lengths) else np.zeros(0, np.float32)
    carry = (rng.standard_normal((len(lengths), 800)) * 0.1).astype(np.float32)
    for use_carry in (False, True):
        print(f"case: ragged clips {lengths} carry={use_carry}", flush=True)
        lm, lv = P.gpu_frames(ctx, P.to_dev(flat), lengths, carry=P.to_dev(carry) if use_carry else None)
        ora_lm = np.concatenate([o.log_mel(clips[c], carry[c] if use_carry else None) for c in range(len(lengths))])
        assert lm.shape == ora_lm.shape == (sum(n // 800 for n in lengths), 80)
        P.check_logmel(lm, ora_lm)
        P.check_levels(lv, ora_lm, o.quantize(ora_lm), gpu_lm=lm)


@pytest.mark.parametrize("so", [[-1000, -200, 7600], [600, 1400, 8800]])
def test_offsets_outside_the_audio(env, so):
    # Offsets that do not describe the audio (clips starting before sample 0,
    # a clip ending past the last sample; 10 frames over 8000 samples, as many
    # as the host accepts): the kernels bounds-check every sample of such
    # frames and read samples outside the audio as zeros, so each clip gives
    # the log-mel of its zero-extended copy.
    dm, ctx = env
    rng = np.random.default_rng(41)
    n_total = 8000
    audio = (rng.standard_normal(n_total) * 0.1).astype(np.float32)
    fo = [0, (so[1] - so[0]) // 800, (so[1] - so[0]) // 800 + (so[2] - so[1]) // 800]
    T = fo[-1]

    def extended(a, b):
        out = np.zeros(b - a, np.float32)
        lo, hi = max(a, 0), min(b, n_total)
        if hi > lo:
            out[lo - a:hi - a] = audio[lo:hi]
        return out

    clips = [extended(so[0], so[1]), extended(so[1], so[2])]
    carry = (rng.standard_normal((2, 800)) * 0.1).astype(np.float32)
    so_d = torch.tensor(so, dtype=torch.int64, device="cuda")
    fo_d = torch.tensor(fo, dtype=torch.int64, device="cuda")
    for use_carry in (False, True):
        print(f"case: offsets {so} around {n_total} samples, carry={use_carry}", flush=True)
        lm = torch.empty((T, 80), dtype=torch.float32, device="cuda")
        lv = torch.empty((T, 80), dtype=torch.uint8, device="cuda")
        c = P.to_dev(carry) if use_carry else None
        dm.dmel_frames(ctx, P.to_dev(audio), n_total, so_d, fo_d, 2, T, c, lm)
        dm.dmel_levels(ctx, P.to_dev(audio), n_total, so_d, fo_d, 2, T, c, lv)
        torch.cuda.synchronize()
        ora_lm = np.concatenate([o.log_mel(clips[k], carry[k] if use_carry else None) for k in range(2)])
        lm_np, lv_np = lm.cpu().numpy(), lv.cpu().numpy()
        P.check_logmel(lm_np, ora_lm)
        P.check_levels(lv_np, ora_lm, o.quantize(ora_lm), gpu_lm=lm_np)


def test_streaming_equals_batch(env, table):
    dm, ctx = env
    S, K = 37, 12
    x = synth.bursts_clips(seed=3, n_clips=S, n_samples=800 * K).cuda()
    so, fo, T = P.offsets([800 * K] * S)
    batch_lv = torch.empty((T, 80), dtype=torch.uint8, device="cuda")
    dm.dmel_levels(ctx, x.reshape(-1), x.numel(), so, fo, S, T, None, batch_lv)
    tab = table.cuda()
    batch_out = torch.empty((T, 6144), dtype=torch.int16, device="cuda")
    dm.dmel_embed(batch_lv, T, tab, 6144, None, None, batch_out, dm.DMEL_BF16, 6144)
    sso, sfo, _ = P.offsets([800] * S)
    ws = torch.empty(dm.dmel_forward_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    carry = torch.zeros((S, 800), dtype=torch.float32, device="cuda")
    step_out = torch.empty((S, 6144), dtype=torch.int16, device="cuda")
    batch_out_v = batch_out.view(S, K, 6144)
    for k in range(K):
        hop = x[:, 800 * k: 800 * (k + 1)].contiguous()
        dm.dmel_forward(ctx, hop.reshape(-1), hop.numel(), sso, sfo, S, S, carry, tab, 6144, None, None, 1e-6,
                        step_out, dm.DMEL_BF16, 6144, None, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.equal(step_out, batch_out_v[:, k]), f"step {k}"
        carry = hop
    # and the stream frames agree with the oracle
    xs = x.cpu().numpy()
    lv_all = batch_lv.cpu().numpy().reshape(S, K, 80)
    for s in (0, S - 1):
        ora_lm = o.log_mel(xs[s])
        P.check_levels(lv_all[s], ora_lm, o.quantize(ora_lm))


def test_frontend_position_invariance(env):
    """A frame's log-mel bits do not depend on where it falls in the kernel's
    16-frame workgroups (its 32-thread group, its wavefront, its 8-frame half
    and the filter slots that read it): the clip is run alone and behind a
    first clip of k = 1..17 frames, which moves every frame through every
    position.  An LDS race between the frames or wavefronts of a workgroup
    would show up as a difference."""
    dm, ctx = env
    x = synth.bursts_clips(seed=21, n_clips=1, n_samples=800 * 61).reshape(-1).cuda()
    so, fo, T = P.offsets([x.numel()])
    ref = torch.empty((T, 80), dtype=torch.float32, device="cuda")
    dm.dmel_frames(ctx, x, x.numel(), so, fo, 1, T, None, ref)
    pre = synth.bursts_clips(seed=22, n_clips=1, n_samples=800 * 17).reshape(-1).cuda()
    for k in range(1, 18):
        a = torch.cat([pre[: 800 * k], x])
        so2, fo2, T2 = P.offsets([800 * k, x.numel()])
        lm = torch.empty((T2, 80), dtype=torch.float32, device="cuda")
        dm.dmel_frames(ctx, a, a.numel(), so2, fo2, 2, T2, None, lm)
        torch.cuda.synchronize()
        assert torch.equal(lm[k:].view(torch.int32), ref.view(torch.int32)), f"prefix of {k} frames"


def test_determinism_and_out_rows(env, table):
    dm, ctx = env
    rng = np.random.default_rng(41)
    n, d = 700, 6144
    lv = P.to_dev(rng.integers(0, 16, size=(n, 80)).astype(np.uint8))
    tab = table.cuda()
    a = torch.empty((n, d), dtype=torch.int16, device="cuda")
    b = torch.empty((n, d), dtype=torch.int16, device="cuda")
    dm.dmel_embed(lv, n, tab, d, None, None, a, dm.DMEL_BF16, d)
    dm.dmel_embed(lv, n, tab, d, None, None, b, dm.DMEL_BF16, d)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # scatter into a wider, larger buffer through out_rows
    stride = d + 64
    rows = torch.from_numpy(rng.permutation(2 * n)[:n].astype(np.int64)).cuda()
    big = torch.full((2 * n, stride), 0x7777, dtype=torch.int16, device="cuda")
    dm.dmel_embed(lv, n, tab, d, None, None, big, dm.DMEL_BF16, stride, rows)
    torch.cuda.synchronize()
    assert torch.equal(big[rows, :d], a)
    untouched = torch.ones(2 * n, dtype=torch.bool, device="cuda")
    untouched[rows] = False
    assert bool((big[untouched] == 0x7777).all()) and bool((big[:, d:] == 0x7777).all())


def test_gather_rows(env):
    dm, ctx = env
    rng = np.random.default_rng(51)
    V, d, n = 1000, 128, 333
    text = synth.table_bf16(seed=9, rows=V, d_model=d).cuda()
    ids = rng.integers(-5, V + 5, size=n).astype(np.int32)
    rows = rng.permutation(n + 10)[:n].astype(np.int64)
    out = torch.full((n + 10, d), 0x1234, dtype=torch.int16, device="cuda")
    dm.dmel_gather_rows(text, V, d, P.to_dev(ids), n, out, d, P.to_dev(rows))
    torch.cuda.synchronize()
    o_np = out.cpu().numpy()
    t_np = text.cpu().numpy()
    for i in range(n):
        want = t_np[ids[i]] if 0 <= ids[i] < V else np.zeros(d, np.int16)
        assert np.array_equal(o_np[rows[i]], want)


def test_gram_and_rms_scale(env, table):
    dm, ctx = env
    tab = table.cuda()
    gram = torch.empty((1280, 1280), dtype=torch.float64, device="cuda")
    dm.dmel_rms_gram(tab, 6144, gram)
    torch.cuda.synchronize()
    E = o.bf16_to_f32(_tbits(table)).astype(np.float64)
    G = E @ E.T
    g = gram.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - G) / (np.abs(G) + 1e-3)) < 1e-11   # fp64 accumulation, stored fp64
    rng = np.random.default_rng(61)
    n = 1500
    lv = rng.integers(0, 16, size=(n, 80)).astype(np.uint8)
    scale = torch.empty(n, dtype=torch.float32, device="cuda")
    dm.dmel_rms_scale(P.to_dev(lv), n, gram, 6144, 1e-6, scale)
    torch.cuda.synchronize()
    s = o.embed_sum(lv, _tbits(table)).astype(np.float64)
    want = 1.0 / np.sqrt(np.mean(s * s, axis=1) + 1e-6)
    rel = np.abs(scale.cpu().numpy() - want) / want
    assert rel.max() < 1e-6, rel.max()


def test_silence_and_empty(env, table):
    dm, ctx = env
    x = np.zeros(800 * 9 + 17, np.float32)
    lm, lv = P.gpu_frames(ctx, P.to_dev(x), [x.size])
    assert np.all(lv == 0)
    got = P.gpu_embed(lv, table, 6144, out_dtype="f32")
    want = o.embed_sum(np.zeros((1, 80), np.uint8), _tbits(table))[0]
    assert np.array_equal(got, np.broadcast_to(want, got.shape))
    # no frames: a valid no-op
    so, fo, T = P.offsets([799])
    assert T == 0
    out = torch.full((1, 6144), 5, dtype=torch.int16, device="cuda")
    dm.dmel_forward(ctx, P.to_dev(np.zeros(799, np.float32)), 799, so, fo, 1, 0, None, table.cuda(), 6144,
                    None, None, 1e-6, out, dm.DMEL_BF16, 6144, None, None, 0)
    torch.cuda.synchronize()
    assert bool((out == 5).all())


def test_scale_and_embed_independent_of_batch_size(env, table):
    """Small batches take the direct RMSNorm-scale kernel and a different
    strips-per-workgroup choice; a token's result must not depend on that."""
    dm, ctx = env
    rng = np.random.default_rng(71)
    n_big = 131072 + 3001          # above the direct-kernel limit: staged Gram kernel
    n_small = 4096
    lv = P.to_dev(rng.integers(0, 16, size=(n_big, 80)).astype(np.uint8))
    tab = table.cuda()
    gram = torch.empty((1280, 1280), dtype=torch.float64, device="cuda")
    dm.dmel_rms_gram(tab, 6144, gram)
    s_big = torch.empty(n_big, dtype=torch.float32, device="cuda")
    s_small = torch.empty(n_small, dtype=torch.float32, device="cuda")
    dm.dmel_rms_scale(lv, n_big, gram, 6144, 1e-6, s_big)
    dm.dmel_rms_scale(lv, n_small, gram, 6144, 1e-6, s_small)
    # the ragged last workgroups of the staged kernel against the direct one
    s_tail = torch.empty(n_small, dtype=torch.float32, device="cuda")
    dm.dmel_rms_scale(lv[n_big - n_small:], n_small, gram, 6144, 1e-6, s_tail)
    torch.cuda.synchronize()
    assert torch.equal(s_small, s_big[:n_small])
    assert torch.equal(s_tail, s_big[n_big - n_small:])
    s = o.embed_sum(lv[:300].cpu().numpy(), _tbits(table)).astype(np.float64)
    want = 1.0 / np.sqrt(np.mean(s * s, axis=1) + 1e-6)
    assert np.max(np.abs(s_big[:300].cpu().numpy() - want) / want) < 1e-6
    w = torch.ones(6144, dtype=torch.float32, device="cuda")
    a = torch.empty((20000, 6144), dtype=torch.int16, device="cuda")
    b = torch.empty((n_small, 6144), dtype=torch.int16, device="cuda")
    dm.dmel_embed(lv, 20000, tab, 6144, w, s_big, a, dm.DMEL_BF16, 6144)
    dm.dmel_embed(lv, n_small, tab, 6144, w, s_small, b, dm.DMEL_BF16, 6144)
    torch.cuda.synchronize()
    assert torch.equal(a[:n_small], b)


@pytest.mark.parametrize("cfg", [None, {"n_mel_bins": 40, "mel_vocab_size": 8, "min_value": -5.0, "max_value": 1.0}])
def test_forward_rmsnorm_small_batch_paths(env, table, cfg):
    """dmel_forward on a small batch takes the bin-parallel RMSNorm-scale path
    (its workspace holds the partial sums); the same tokens through
    dmel_levels -> dmel_rms_scale (direct kernel) -> dmel_embed, and the
    staged kernel on a batch above the small-batch limit, give the same bits."""
    dm, ctx0 = env
    ctx = ctx0 if cfg is None else dm.dmel_create_config(0, cfg)
    try:
        nb = 80 if cfg is None else cfg["n_mel_bins"]
        nl = 16 if cfg is None else cfg["mel_vocab_size"]
        print(f"case: forward with RMSNorm, small batch, config {cfg}", flush=True)
        x = synth.bursts_clips(seed=5, n_clips=6, n_samples=480000).cuda()
        so, fo, T = P.offsets([480000] * 6)
        tab = (table if cfg is None else synth.table_bf16(seed=78, rows=nb * nl, d_model=6144)).cuda()
        gram = torch.empty((1280, 1280), dtype=torch.float64, device="cuda")
        dm.dmel_rms_gram(tab, 6144, gram, n_bins=nb, n_levels=nl)
        w = (torch.rand(6144, generator=torch.Generator().manual_seed(5)) + 0.5).cuda()
        out = torch.empty((T, 6144), dtype=torch.int16, device="cuda")
        ws = torch.empty(dm.dmel_forward_workspace_bytes(T), dtype=torch.uint8, device="cuda")
        dm.dmel_forward(ctx, x.reshape(-1), x.numel(), so, fo, 6, T, None, tab, 6144, w, gram, 1e-6, out,
                        dm.DMEL_BF16, 6144, None, ws, ws.numel())
        lv = torch.empty((T, nb), dtype=torch.uint8, device="cuda")
        dm.dmel_levels(ctx, x.reshape(-1), x.numel(), so, fo, 6, T, None, lv)
        sc = torch.empty(T, dtype=torch.float32, device="cuda")
        dm.dmel_rms_scale(lv, T, gram, 6144, 1e-6, sc, n_bins=nb, n_levels=nl)
        ref = torch.empty((T, 6144), dtype=torch.int16, device="cuda")
        dm.dmel_embed(lv, T, tab, 6144, w, sc, ref, dm.DMEL_BF16, 6144, n_bins=nb, n_levels=nl)
        # the staged kernel: the same levels repeated past the small-batch limit
        reps = 131072 // T + 1
        big = lv.repeat(reps, 1)
        sc_big = torch.empty(big.shape[0], dtype=torch.float32, device="cuda")
        dm.dmel_rms_scale(big, big.shape[0], gram, 6144, 1e-6, sc_big, n_bins=nb, n_levels=nl)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(sc, sc_big[:T])
        # the forward's scales sit in its workspace after the levels
        off = (T * 80 + 255) // 256 * 256
        assert torch.equal(ws[off: off + 4 * T].view(torch.float32), sc)
    finally:
        if cfg is not None:
            torch.cuda.synchronize()
            dm.dmel_destroy(ctx)
