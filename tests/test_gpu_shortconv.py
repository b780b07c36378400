"""GPU parity of the short convolution (width 4, residual, per-request state)
through the C ABI against the fp64 oracle on the same seeded inputs.

Bars: the state is exact (it holds inputs); fp32 output within
tol = 2^-21 * (|x[t]| + sum_d |w_d x[t-d]|) of the exact value (five fp32
roundings of partial sums bounded by that magnitude, with margin); bf16
output between the nearest-even roundings of exact - tol and exact + tol
(rounding is monotone, so the rounding of any fp32 value within tol lies
there; it differs from the rounding of the exact value only next to a
midpoint).  Chunked and one-token-per-step
processing with the state carried equals one pass bit for bit."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import dmel_oracle as o
from oracle import shortconv_oracle as sc
from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from encoder_free_audio_amd import dmel
    return dmel


def _off(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def run_gpu(dm, x, lengths, w, state=None, y_dtype="bf16", with_state_out=True):
    """x: int16 tensor [T, C] (bf16 bits); returns (y numpy, state_out numpy or None)."""
    T, C = x.shape
    S = len(lengths)
    off = torch.from_numpy(_off(lengths)).cuda()
    xd = x.cuda()
    wd = w.cuda()
    sin = state.cuda() if state is not None else None
    sout = torch.full((max(S, 1), 3, C), 0x7FC1, dtype=torch.int16, device="cuda") if with_state_out else None
    dt = dm.DMEL_BF16 if y_dtype == "bf16" else dm.DMEL_F32
    y = torch.empty((max(T, 1), C), dtype=torch.int16 if dt == dm.DMEL_BF16 else torch.float32, device="cuda")
    dm.dmel_shortconv(xd, T, C, off, S, wd, sin, sout, y, dt)
    torch.cuda.synchronize()
    yn = y[:T].cpu().numpy()
    return (yn.view(np.uint16) if dt == dm.DMEL_BF16 else yn), (sout[:S].cpu().numpy().view(np.uint16) if with_state_out else None)


def check_y(got, x_bits, lengths, w, state_bits, y_dtype):
    off = _off(lengths)
    exact, st = sc.shortconv(x_bits, off, w, state_bits)
    # magnitude of the terms: the same formula on |x| and |w|
    xa = (x_bits & np.uint16(0x7FFF)).astype(np.uint16)
    sa = None if state_bits is None else (state_bits & np.uint16(0x7FFF)).astype(np.uint16)
    mag, _ = sc.shortconv(xa, off, np.abs(w), sa)
    tol = 2.0 ** -21 * mag
    if y_dtype == "f32":
        err = np.abs(got.astype(np.float64) - exact)
        assert np.all(err <= tol), f"max excess {np.max(err - tol)}"
        return st, 0
    want = o.f64_to_bf16(exact)
    lo = o.bf16_to_f32(o.f64_to_bf16(exact - tol)).astype(np.float64)
    hi = o.bf16_to_f32(o.f64_to_bf16(exact + tol)).astype(np.float64)
    gv = o.bf16_to_f32(got).astype(np.float64)
    bad = (gv < lo) | (gv > hi)
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs outside the rounding of exact +- tol"
    return st, int((got != want).sum())


def test_worked_example(dm, golden_dir):
    with open(os.path.join(golden_dir, "shortconv_worked.json")) as f:
        g = json.load(f)
    C = 8  # the one-channel example in every channel of one 16-byte group
    x = np.repeat(np.array(g["x"], dtype=np.float32), C, axis=1)
    st = np.repeat(np.array(g["state_in"], dtype=np.float32), C, axis=2)
    w = np.repeat(np.array(g["weight"], dtype=np.float32), C, axis=0)
    bits = lambda a: torch.from_numpy((np.ascontiguousarray(a).view(np.uint32) >> 16).astype(np.uint16).view(np.int16))
    lengths = list(np.diff(g["seq_off"]))
    y, so = run_gpu(dm, bits(x), lengths, torch.from_numpy(w), bits(st), y_dtype="f32")
    assert np.array_equal(y, np.repeat(np.array(g["y"], dtype=np.float32), C, axis=1))
    assert np.array_equal(o.bf16_to_f32(so), np.repeat(np.array(g["state_out"], dtype=np.float32), C, axis=2))


@pytest.mark.parametrize("C", [8, 64, 2056, 6144])
@pytest.mark.parametrize("with_state", [False, True])
def test_ragged_requests(dm, C, with_state):
    lengths = [0, 1, 2, 3, 4, 5, 7, 31, 32, 33, 100, 0, 0, 257, 1]
    print(f"case: shortconv ragged requests C={C} state={with_state}", flush=True)
    T = sum(lengths)
    x = synth.activations_bf16(seed=C + 1, n_tokens=T, channels=C)
    w = synth.shortconv_weight(seed=C + 2, channels=C)
    st = synth.activations_bf16(seed=C + 3, n_tokens=len(lengths) * 3, channels=C).view(len(lengths), 3, C) \
        if with_state else None
    xb = x.numpy().view(np.uint16)
    sb = st.numpy().view(np.uint16) if st is not None else None
    for dt in ("f32", "bf16"):
        y, so = run_gpu(dm, x, lengths, w, st, y_dtype=dt)
        want_state, nd = check_y(y, xb, lengths, w.numpy().astype(np.float64), sb, dt)
        assert np.array_equal(so, want_state)
    print(f"bf16 midpoint differences: {nd}")


@pytest.mark.parametrize("avg", [1, 3, 9, 40, 300])
def test_run_lengths_and_many_requests(dm, avg):
    # the kernel's run length follows the average request length; empty
    # requests fall at run boundaries, inside runs and at the end
    rng = np.random.default_rng(avg)
    n = 400
    lengths = [int(v) for v in rng.integers(0, 2 * avg + 1, n)]
    lengths[0] = 0
    lengths[-3:] = [0, 0, 0]
    C = 16
    T = sum(lengths)
    print(f"case: {n} requests, mean length {avg}, T={T}", flush=True)
    x = synth.activations_bf16(seed=50 + avg, n_tokens=T, channels=C)
    w = synth.shortconv_weight(seed=51, channels=C)
    st = synth.activations_bf16(seed=52, n_tokens=n * 3, channels=C).view(n, 3, C)
    y, so = run_gpu(dm, x, lengths, w, st, y_dtype="f32")
    want_state, _ = check_y(y, x.numpy().view(np.uint16), lengths, w.numpy().astype(np.float64),
                            st.numpy().view(np.uint16), "f32")
    assert np.array_equal(so, want_state)


def test_decode_steps_equal_one_pass(dm):
    # S requests, K steps of one token each, the state carried in two buffers
    S, K, C = 300, 40, 256
    print(f"case: decode {S} requests x {K} steps, C={C}", flush=True)
    x = synth.activations_bf16(seed=60, n_tokens=S * K, channels=C).cuda().view(S, K, C)
    w = synth.shortconv_weight(seed=61, channels=C).cuda()
    st0 = synth.activations_bf16(seed=62, n_tokens=S * 3, channels=C).cuda().view(S, 3, C)
    off_all = torch.from_numpy(_off([K] * S)).cuda()
    y_all = torch.empty((S * K, C), dtype=torch.int16, device="cuda")
    st_all = torch.empty((S, 3, C), dtype=torch.int16, device="cuda")
    dm.dmel_shortconv(x.reshape(S * K, C), S * K, C, off_all, S, w, st0, st_all, y_all, dm.DMEL_BF16)
    off1 = torch.from_numpy(_off([1] * S)).cuda()
    bufs = [st0.clone(), torch.empty_like(st0)]
    y_step = torch.empty((S, C), dtype=torch.int16, device="cuda")
    for k in range(K):
        xk = x[:, k, :].contiguous()
        dm.dmel_shortconv(xk, S, C, off1, S, w, bufs[k % 2], bufs[(k + 1) % 2], y_step, dm.DMEL_BF16)
        assert torch.equal(y_step, y_all.view(S, K, C)[:, k]), f"step {k}"
    torch.cuda.synchronize()
    assert torch.equal(bufs[K % 2], st_all)


def test_chunked_prefill_equals_one_pass(dm):
    C, n = 512, 5000
    cuts = [0, 1, 2, 33, 1000, 1001, 4096, 5000]
    print(f"case: chunked prefill C={C} n={n}", flush=True)
    x = synth.activations_bf16(seed=70, n_tokens=n, channels=C).cuda()
    w = synth.shortconv_weight(seed=71, channels=C).cuda()
    off = torch.tensor([0, n], dtype=torch.int64, device="cuda")
    y_all = torch.empty((n, C), dtype=torch.int16, device="cuda")
    st_all = torch.empty((1, 3, C), dtype=torch.int16, device="cuda")
    dm.dmel_shortconv(x, n, C, off, 1, w, None, st_all, y_all, dm.DMEL_BF16)
    bufs = [torch.zeros((1, 3, C), dtype=torch.int16, device="cuda"), torch.empty((1, 3, C), dtype=torch.int16,
                                                                                   device="cuda")]
    for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        yk = torch.empty((max(b - a, 1), C), dtype=torch.int16, device="cuda")
        offk = torch.tensor([0, b - a], dtype=torch.int64, device="cuda")
        dm.dmel_shortconv(x[a:b].contiguous(), b - a, C, offk, 1, w, bufs[i % 2], bufs[(i + 1) % 2], yk,
                          dm.DMEL_BF16)
        assert torch.equal(yk[: b - a], y_all[a:b]), (a, b)
    torch.cuda.synchronize()
    assert torch.equal(bufs[(len(cuts) - 1) % 2], st_all)


def test_empty_batch_passes_states(dm):
    C, S = 24, 5
    st = synth.activations_bf16(seed=80, n_tokens=S * 3, channels=C).cuda().view(S, 3, C)
    out = torch.empty_like(st)
    off = torch.zeros(S + 1, dtype=torch.int64, device="cuda")
    w = synth.shortconv_weight(seed=81, channels=C).cuda()
    dm.dmel_shortconv(None, 0, C, off, S, w, st, out, None, dm.DMEL_BF16)
    torch.cuda.synchronize()
    assert torch.equal(out, st)
    # and with no input state: zeros
    dm.dmel_shortconv(None, 0, C, off, S, w, None, out, None, dm.DMEL_BF16)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0


def test_full_size_prefill_sampled(dm):
    # 64 requests x 24,000 tokens x 6144 channels (the audio tokens of
    # 64 x 20 min clips), state in and out, sampled rows against the oracle
    S, L, C = 64, 24000, 6144
    T = S * L
    print("case: shortconv 64 x 24000 x 6144 bf16", flush=True)
    x = synth.activations_bf16(seed=90, n_tokens=T, channels=C, device="cuda")
    w = synth.shortconv_weight(seed=91, channels=C)
    st = synth.activations_bf16(seed=92, n_tokens=S * 3, channels=C, device="cuda").view(S, 3, C)
    off = torch.from_numpy(_off([L] * S)).cuda()
    y = torch.empty((T, C), dtype=torch.int16, device="cuda")
    so = torch.empty((S, 3, C), dtype=torch.int16, device="cuda")
    dm.dmel_shortconv(x, T, C, off, S, w.cuda(), st, so, y, dm.DMEL_BF16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(93)
    picks = [(int(s), int(t)) for s, t in zip(rng.integers(0, S, 40), rng.integers(0, L, 40))]
    picks += [(0, 0), (0, 1), (0, 2), (63, L - 1), (17, 0)]
    wn = w.numpy().astype(np.float64)
    for s, t in picks:
        a = s * L
        stb = st[s].cpu().numpy().view(np.uint16)
        # the three inputs before token t: token rows, or the request's state
        prev = np.stack([x[a + t - d].cpu().numpy().view(np.uint16) if t - d >= 0 else stb[3 + t - d]
                         for d in (3, 2, 1)])
        xt = x[a + t: a + t + 1].cpu().numpy().view(np.uint16)
        got = y[a + t: a + t + 1].cpu().numpy().view(np.uint16)
        check_y(got, xt, [1], wn, prev[None], "bf16")
    # the states: the last three inputs of each request
    assert torch.equal(so, x.view(S, L, C)[:, L - 3:, :])
