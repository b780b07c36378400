"""GPU parity of the hMLP image front end through the C ABI.

* Each stage (dmel_hmlp_stage: y = x W^T + b, GELU on stages 1-3) against the
  oracle's stage evaluated exactly on the same bf16 input.  Bar: the GPU's
  fp32 result within tol = 2 K 2^-24 (sum_k |x_k w_k| + |b|) of the exact
  pre-activation (K fp32 roundings of partial sums bounded by that
  magnitude, doubled for the matrix cores' internal order), so the GELU output
  within 1.13 tol (|GELU'| <= 1.13) + 2^-21 |g| (fp32 erf); fp32 output inside
  that band, bf16 output between the nearest-even roundings of its ends.
* The stage inputs of the GPU chain, read back as images of stage outputs,
  agree with the oracle's 5 x 5 sub-patch and 2 x 2 merge definitions (this
  pins the Morton row order the kernels use against the spatial definition).
* dmel_hmlp_forward equals the chain of its four stages bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import hmlp_oracle as ho
from oracle import dmel_oracle as o
from encoder_free_audio_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from encoder_free_audio_amd import dmel
    return dmel


def morton_order():
    """(y, x) of the 64 Morton positions of an 8 x 8 grid (bits y2 x2 y1 x1 y0 x0)."""
    ys, xs = [], []
    for m in range(64):
        y = x = 0
        for b in range(3):
            x |= ((m >> (2 * b)) & 1) << b
            y |= ((m >> (2 * b + 1)) & 1) << b
        ys.append(y)
        xs.append(x)
    return np.array(ys), np.array(xs)


def make_weights(seed, hidden, d, device="cuda"):
    rng = np.random.default_rng(seed)
    shapes = [(hidden, 75), (hidden, 4 * hidden), (hidden, 4 * hidden), (d, 4 * hidden)]
    ws = []
    for n, k in shapes:
        w = synth.table_bf16(seed=int(rng.integers(1 << 30)), rows=n, d_model=k, std=1.0 / np.sqrt(k))
        b = torch.from_numpy((rng.standard_normal(n) * 0.1).astype(np.float32))
        ws.append((w.to(device), b.to(device)))
    return ws


def a1_from_images(images, n, H, W):
    """Stage-1 input rows in the kernels' order: patches row-major, sub-patches in Morton order, K padded to 96."""
    ph, pw = H // 40, W // 40
    x = images.view(n, ph, 8, 5, pw, 8, 5, 3).permute(0, 1, 4, 2, 5, 3, 6, 7).reshape(n * ph * pw, 8, 8, 75)
    ys, xs = morton_order()
    a = x[:, torch.from_numpy(ys).to(x.device), torch.from_numpy(xs).to(x.device), :].reshape(-1, 75)
    out = torch.zeros((a.shape[0], 96), dtype=torch.int16, device=x.device)
    out[:, :75] = a
    return out


def gpu_chain(dm, a1, ws, hidden, d, P):
    w1p = torch.zeros((hidden, 96), dtype=torch.int16, device="cuda")
    w1p[:, :75] = ws[0][0]
    h1 = torch.empty((P * 64, hidden), dtype=torch.int16, device="cuda")
    h2 = torch.empty((P * 16, hidden), dtype=torch.int16, device="cuda")
    h3 = torch.empty((P * 4, hidden), dtype=torch.int16, device="cuda")
    y = torch.empty((P, d), dtype=torch.float32, device="cuda")
    dm.dmel_hmlp_stage(a1, P * 64, 96, w1p, ws[0][1], hidden, 1, h1, dm.DMEL_BF16)
    dm.dmel_hmlp_stage(h1, P * 16, 4 * hidden, ws[1][0], ws[1][1], hidden, 1, h2, dm.DMEL_BF16)
    dm.dmel_hmlp_stage(h2, P * 4, 4 * hidden, ws[2][0], ws[2][1], hidden, 1, h3, dm.DMEL_BF16)
    dm.dmel_hmlp_stage(h3, P, 4 * hidden, ws[3][0], ws[3][1], d, 0, y, dm.DMEL_F32)
    torch.cuda.synchronize()
    return w1p, h1, h2, h3, y


def check_stage(x_bits, w_bits, bias, got, gelu, out_bf16):
    x = ho.bf16_bits_to_f64(x_bits)
    w = ho.bf16_bits_to_f64(w_bits)
    b = np.asarray(bias, dtype=np.float64)
    pre = x @ w.T + b
    k = x.shape[1]
    tol = 2.0 * k * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T + np.abs(b))
    if gelu:
        g = ho.gelu(pre)
        tol = 1.13 * tol + 2.0 ** -21 * np.abs(g) + 1e-30
    else:
        g = pre
        tol = tol + 1e-30
    if out_bf16:
        lo = ho.f64_to_bf16_value(g - tol)
        hi = ho.f64_to_bf16_value(g + tol)
        gv = ho.bf16_bits_to_f64(got)
        bad = (gv < lo) | (gv > hi)
    else:
        bad = np.abs(np.asarray(got, np.float64) - g) > tol
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} outside the bar"


def to_spatial(rows, n, H, W, level):
    """Stage outputs [P * 4**(3-level) ... , C] in the kernels' order -> [n, side_h, side_w, C] images.

    level 1: 8 x 8 per patch (Morton), 2: 4 x 4, 3: 2 x 2."""
    side = {1: 8, 2: 4, 3: 2}[level]
    ph, pw = H // 40, W // 40
    C = rows.shape[1]
    per = rows.reshape(n, ph, pw, side * side, C)
    ys, xs = morton_order()
    # Morton index at a coarser level: positions of the 8 x 8 order grouped by 4**(level-1)
    grp = 4 ** (level - 1)
    ys_l, xs_l = ys[::grp] // (8 // side), xs[::grp] // (8 // side)
    out = np.zeros((n, ph, side, pw, side, C), dtype=rows.dtype)
    for m in range(side * side):
        out[:, :, ys_l[m], :, xs_l[m], :] = per[:, :, :, m, :]
    return out.reshape(n, ph * side, pw * side, C)


@pytest.mark.parametrize("M,K,N", [(300, 96, 128), (128 * 3 + 5, 6144, 256), (64, 512, 1536), (1, 32, 128),
                                   (1000, 192, 768), (257, 64, 512), (2048, 128, 1792)])
@pytest.mark.parametrize("gelu", [0, 1])
def test_stage_gemm(dm, M, K, N, gelu):
    print(f"case: stage GEMM M={M} K={K} N={N} gelu={gelu}", flush=True)
    rng = np.random.default_rng(M + K + N + gelu)
    x = synth.table_bf16(seed=int(rng.integers(1 << 30)), rows=M, d_model=K, std=1.0).cuda()
    w = synth.table_bf16(seed=int(rng.integers(1 << 30)), rows=N, d_model=K, std=1.0 / np.sqrt(K)).cuda()
    b = torch.from_numpy((rng.standard_normal(N) * 0.1).astype(np.float32)).cuda()
    for dt in (dm.DMEL_F32, dm.DMEL_BF16):
        y = torch.empty((M, N), dtype=torch.float32 if dt == dm.DMEL_F32 else torch.int16, device="cuda")
        dm.dmel_hmlp_stage(x, M, K, w, b, N, gelu, y, dt)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        check_stage(x.cpu().numpy().view(np.uint16), w.cpu().numpy().view(np.uint16), b.cpu().numpy(),
                    got.view(np.uint16) if dt == dm.DMEL_BF16 else got, gelu, dt == dm.DMEL_BF16)


@pytest.mark.parametrize("n,H,W,hidden,d", [(2, 80, 120, 128, 256), (1, 200, 160, 256, 384)])
def test_forward_small_images(dm, n, H, W, hidden, d):
    print(f"case: hMLP {n} x {H} x {W}, hidden {hidden}, d {d}", flush=True)
    P = ho.num_patches(n, H, W)
    images = synth.table_bf16(seed=H + W, rows=n * H * W, d_model=3, std=1.0).cuda()
    ws = make_weights(H * W + hidden, hidden, d)
    a1 = a1_from_images(images, n, H, W)
    w1p, h1, h2, h3, y = gpu_chain(dm, a1, ws, hidden, d, P)
    # the forward equals the chain of its stages bit for bit
    wsb = dm.dmel_hmlp_workspace_bytes(n, H, W, hidden)
    wsp = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((P, d), dtype=torch.float32, device="cuda")
    flat = [t for pair in ws for t in pair]
    dm.dmel_hmlp_forward(images, n, H, W, *flat, hidden, d, out, dm.DMEL_F32, wsp, wsb)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), y.view(torch.int32))
    # stage inputs agree with the oracle's spatial definitions
    img_np = images.cpu().numpy().view(np.uint16).reshape(n, H, W, 3)
    sub = ho.subpatches(ho.bf16_bits_to_f64(img_np))                       # [n, H/5, W/5, 75]
    a1_sp = to_spatial(a1.cpu().numpy()[:, :75].view(np.uint16), n, H, W, 1)
    assert np.array_equal(ho.bf16_bits_to_f64(a1_sp), sub)
    h_np = [t.cpu().numpy().view(np.uint16) for t in (h1, h2, h3)]
    for lvl in (1, 2):
        merged = ho.merge2x2(to_spatial(h_np[lvl - 1], n, H, W, lvl))     # oracle's merge of the GPU's outputs
        nxt_in = h_np[lvl - 1].reshape(-1, 4 * hidden)                    # the kernels' next-stage input rows
        assert np.array_equal(to_spatial(nxt_in, n, H, W, lvl + 1), merged)
    # each stage against the oracle's stage on the GPU's own input
    wn = [(w.cpu().numpy().view(np.uint16), b.cpu().numpy()) for w, b in ws]
    check_stage(a1.cpu().numpy().view(np.uint16)[:, :75], wn[0][0], wn[0][1], h_np[0], True, True)
    check_stage(h_np[0].reshape(-1, 4 * hidden), wn[1][0], wn[1][1], h_np[1], True, True)
    check_stage(h_np[1].reshape(-1, 4 * hidden), wn[2][0], wn[2][1], h_np[2], True, True)
    check_stage(h_np[2].reshape(-1, 4 * hidden), wn[3][0], wn[3][1], y.cpu().numpy(), False, False)
    # and the whole stem against the oracle, loosely (hidden bf16 roundings may differ next to midpoints)
    ref = ho.hmlp(img_np, wn)
    rel = np.max(np.abs(y.cpu().numpy() - ref)) / np.max(np.abs(ref))
    print(f"end-to-end max relative deviation {rel:.2e}")
    assert rel < 2e-2


def test_forward_full_size_sampled(dm):
    # 8 images of 1280 x 1280 (8192 patches), hidden 1536, d 6144, bf16 out
    n, H, W, hidden, d = 8, 1280, 1280, 1536, 6144
    print("case: hMLP 8 x 1280 x 1280", flush=True)
    P = ho.num_patches(n, H, W)
    images = synth.table_bf16(seed=5, rows=n * H * W, d_model=3, std=1.0, device="cuda")
    ws = make_weights(6, hidden, d)
    a1 = a1_from_images(images, n, H, W)
    w1p, h1, h2, h3, y = gpu_chain(dm, a1, ws, hidden, d, P)
    wsb = dm.dmel_hmlp_workspace_bytes(n, H, W, hidden)
    wsp = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((P, d), dtype=torch.float32, device="cuda")
    flat = [t for pair in ws for t in pair]
    dm.dmel_hmlp_forward(images, n, H, W, *flat, hidden, d, out, dm.DMEL_F32, wsp, wsb)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), y.view(torch.int32))
    wn = [(w.cpu().numpy().view(np.uint16), b.cpu().numpy()) for w, b in ws]
    rng = np.random.default_rng(7)
    for p in list(rng.integers(0, P, 3)) + [0, P - 1]:
        p = int(p)
        r1 = slice(p * 64, p * 64 + 64)
        check_stage(a1[r1].cpu().numpy().view(np.uint16)[:, :75], wn[0][0], wn[0][1],
                    h1[r1].cpu().numpy().view(np.uint16), True, True)
        x2 = h1[r1].cpu().numpy().view(np.uint16).reshape(16, 4 * hidden)
        check_stage(x2, wn[1][0], wn[1][1], h2[p * 16: p * 16 + 16].cpu().numpy().view(np.uint16), True, True)
        x3 = h2[p * 16: p * 16 + 16].cpu().numpy().view(np.uint16).reshape(4, 4 * hidden)
        check_stage(x3, wn[2][0], wn[2][1], h3[p * 4: p * 4 + 4].cpu().numpy().view(np.uint16), True, True)
        x4 = h3[p * 4: p * 4 + 4].cpu().numpy().view(np.uint16).reshape(1, 4 * hidden)
        check_stage(x4, wn[3][0], wn[3][1], y[p: p + 1].cpu().numpy(), False, False)
