"""Benchmark of the dMel front end on one MI355X.

One step = one dmel_forward call, the whole hot path over one batch: framing
+ FFT + log-mel + quantizer, the RMSNorm scales and the bag-of-bins embedding
with RMSNorm and bf16 output, for 64 clips of 20 minutes of speech-like 16 kHz
audio (1,536,000 tokens of width 6144).  Inputs are generated on the device
before the timed region; the table's Gram matrix is computed once per table,
outside it.  After the timed region the same three launches are called one by
one with events between them for the per-kernel split, and the oracle runs on
a sample of the batch, compared with the GPU's results for it.

Prints one JSON line (see the fields below).  ``--gpus N`` with N > 1 exits:
this front end runs on one GPU here.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from encoder_free_audio_amd import dmel as dm  # noqa: E402
from encoder_free_audio_amd import synth  # noqa: E402

HBM_BYTES_PER_TOKEN = 800 * 4 + 6144 * 2    # 3,200 B audio read (800 new samples) + 12,288 B bf16 token write
# fp32 adds: the chip's fp32 vector figure (157.3 TFLOP/s) is 128 fused multiply-adds per clock per CU at
# 2.4 GHz; an add is one flop, so 256 CUs x 128 x 2.4 GHz = 78.6 T adds/s.  Plain (non-packed) v_add_f32
# with VGPR operands issues at 64.6 T/s (VOP2) to 70.2 T/s (VOP3) on this chip: bench.py --workload valu,
# profiles/valu_rates_mi355x.md.
PEAK_ADD_TFLOPS = 78.6
PEAK_HBM_GBPS = 8000.0
# LDS: ds_read_b128 of 16-float rows at the embedding's 80-byte pitch, measured on this chip (bench.py --workload
# valu, profiles/valu_rates_mi355x.md): the ceiling of the embedding's gathers, which read 4 bytes per add
LDS_GATHER_TBPS = 143.0
PEAK_FP32_TFLOPS = 157.3        # fp32 vector peak with FMA counted as two flops
# algorithmic flops per frame of the front end: FFT 2.5 N log2 N (N = 1600) 42,575,
# mel 3,142, power 2,403, window 1,600
FRONT_FLOPS_PER_FRAME = 42575 + 3142 + 2403 + 1600
METRIC = "audio tokens/sec (dMel frames→6144-d embeds) + achieved HBM GB/s vs peak"
COUNTERS_MD = os.path.join(ROOT, "profiles", "embed_kernel_64x20min_counters.md")
EMBED_SRCS = [os.path.join(ROOT, "encoder_free_audio_amd", "csrc", f) for f in ("embed.hip", "embed_core.h")]


def embed_traffic():
    """Memory traffic of one embed launch on the 64 x 20 min batch, from the
    committed counter summary - only if embed.hip and embed_core.h are the
    sources that were measured (otherwise the figure would describe another
    kernel)."""
    import hashlib
    import re
    try:
        text = open(COUNTERS_MD).read()
        want = re.search(r"embed.hip \+ embed_core.h sha256: ([0-9a-f]{64})", text).group(1)
        traffic = float(re.search(r"traffic bytes per launch: ([0-9.e+]+)", text).group(1))
        h = hashlib.sha256()
        for f in EMBED_SRCS:
            h.update(open(f, "rb").read())
        have = h.hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    return traffic if have == want else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (batch 20, stream 1000, interleave 5)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--clips", type=int, default=64)
    ap.add_argument("--minutes", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=20000, help="oracle sample: frames per worker")
    ap.add_argument("--workload", choices=("batch", "stream", "interleave", "copy", "shortconv", "shortconv_decode",
                                           "backward", "hmlp", "dft_gemm", "rounding", "valu"),
                    default="batch",
                    help="batch: 64 x 20 min clips (default); stream: 4096 streams, one hop per step; "
                         "interleave: 256 x 32768 audio/text positions; copy: a plain 1 GiB device copy "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters); shortconv: the decoder's width-4 "
                         "short convolution over 64 requests x 24,000 tokens x 6144 channels (prefill); "
                         "shortconv_decode: 4096 requests, one token per step, state carried; backward: the "
                         "RMSNorm and table-gradient backward of the 64 x 20 min batch; hmlp: the four-stage "
                         "image front end over 32 images of 1280 x 1280 (32768 patches of 40 x 40); valu: issue "
                         "rates of single vector-ALU instruction forms (the ceiling the embedding's adds are "
                         "priced against)")
    ap.add_argument("--streams", type=int, default=4096)
    ap.add_argument("--config", default=None,
                    help="batch workload with another front-end configuration, "
                         "'n_mel_bins,mel_vocab_size,min_value,max_value' (e.g. 80,16,-1.5,2 for the serving "
                         "code's default clamp minimum); default: the released 80,16,-7,2")
    args = ap.parse_args()
    if args.config is not None:
        f = args.config.split(",")
        if len(f) != 4:
            ap.error("--config needs four comma-separated values")
        args.config = {"n_mel_bins": int(f[0]), "mel_vocab_size": int(f[1]), "min_value": float(f[2]),
                       "max_value": float(f[3])}
    return args


# Host data of the oracle leg, set before the pool forks (the workers read it
# without copies): per sampled clip its audio, and the GPU's log-mel, levels
# and tokens of the same frames.
_ORACLE_DATA: dict = {}


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(audio_dev, clip_len, table_bits, n_clips, frames_per_worker, gpu_sample, config=None):
    """Time the CPU oracle on a bounded sample of the same workload: the first
    frames of several clips (causal framing makes them the clip's first
    frames), one oracle process per core, and compare its results with the
    GPU's for the same frames (gpu_sample(clip, n_frames) -> (log-mel, levels,
    tokens) on the host).  The time is the slowest worker's oracle forward
    alone (not the comparison)."""
    import multiprocessing as mp

    from oracle import dmel_oracle  # noqa: F401  (imported here: test infrastructure)

    host = _host_cores()
    # at most 16 processes: the GPU machine's share of host cores
    workers = max(1, min(host, 16, n_clips))
    n = frames_per_worker * 800
    _ORACLE_DATA.clear()
    _ORACLE_DATA["clips"] = [(audio_dev[c * clip_len: c * clip_len + n].cpu().numpy(),) + gpu_sample(c, frames_per_worker)
                             for c in range(workers)]
    _ORACLE_DATA["table"] = table_bits.cpu().numpy().view(np.uint16)
    _ORACLE_DATA["config"] = config
    ctx = mp.get_context("fork")
    try:
        with ctx.Pool(workers) as pool:
            res = pool.map(_oracle_job, range(workers), chunksize=1)
    finally:
        _ORACLE_DATA.clear()
    tokens = sum(r["tokens"] for r in res)
    dt = max(r["seconds"] for r in res)
    parity = {}
    for r in res:
        for k, v in r["parity"].items():
            parity[k] = max(parity.get(k, 0.0), v) if k.startswith("max_") else parity.get(k, 0) + v
    return {"value": tokens / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"first {frames_per_worker} frames of each of {workers} clips ({tokens} tokens, "
                      f"RMSNorm on, bf16 out), one oracle process per core; the slowest process took {dt:.1f} s",
            "host_cores": host, "cores_used": workers, "cpu_model": _cpu_model()}, parity


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_job(i):
    """One worker: the oracle forward of one clip's sample (timed), then its
    comparison with the GPU's log-mel, levels and tokens of the same frames
    to the parity bars (counted, not asserted)."""
    from threadpoolctl import threadpool_limits

    from oracle import dmel_oracle as o
    seg, lm_g, lv_g, tok_g = _ORACLE_DATA["clips"][i]
    tb = _ORACLE_DATA["table"]
    config = _ORACLE_DATA["config"]
    cfg = o.Config(**config) if config is not None else None
    w = np.ones(tb.shape[1], dtype=np.float32)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        lm, lv, out, exact = o.forward(seg, tb, rms_weight=w, cfg=cfg)
        dt = time.perf_counter() - t0
        cfg = cfg or o.Config()
        lo, hi = cfg.min_value, cfg.max_value
        err = np.abs(np.clip(lm_g.astype(np.float64), lo, hi) - np.clip(lm, lo, hi))
        edges = o.level_edges(lo, hi, cfg.mel_vocab_size)
        band = (np.min(np.abs(lm[..., None] - edges), axis=-1) <= 1e-3) if edges.size else np.zeros(lm.shape, bool)
        mism = lv_g != lv
        same = ~mism.any(axis=1)
        exact_tok = np.all(tok_g == out, axis=1)
        d = (tok_g != out) & same[:, None]
        # a bf16 difference is within the bar if it is one ulp next to a rounding midpoint
        gv = o.bf16_to_f32(tok_g).astype(np.float64)
        wv = o.bf16_to_f32(out).astype(np.float64)
        mid_ok = (np.abs(exact - 0.5 * (gv + wv)) <= 1e-5 * np.abs(exact)) & \
                 (np.abs(tok_g.astype(np.int64) - out.astype(np.int64)) == 1)
    return {"tokens": int(out.shape[0]), "seconds": dt,
            "parity": {"frames": int(lm.shape[0]), "max_err_clamped_logmel": float(err.max(initial=0.0)),
                       "edge_band": int(band.sum()), "forgiven": int((mism & band).sum()),
                       "level_mismatches_outside_band": int((mism & ~band).sum()),
                       "frames_affected": int(mism.any(axis=1).sum()),
                       "tokens_compared": int(same.sum()), "tokens_bit_exact": int((exact_tok & same).sum()),
                       "bf16_midpoint_ulps": int((d & mid_ok).sum()),
                       "bf16_outside_bar": int((d & ~mid_ok).sum())}}


def one_core_baseline():
    """The oracle on one core for the 1 s three-tone clip (20 tokens, no
    RMSNorm) and the 8 x 30 s bursts batch (4800 tokens, RMSNorm on)."""
    from threadpoolctl import threadpool_limits

    from oracle import dmel_oracle as o
    tb = synth.table_bf16(seed=1234).numpy().view(np.uint16)
    res = {}
    with threadpool_limits(1):
        x = synth.tones_clip(seed=0)
        t0 = time.perf_counter()
        _, _, out, _ = o.forward(x, tb)
        res["tones_1s_tokens_per_s"] = out.shape[0] / (time.perf_counter() - t0)
        xs = synth.bursts_clips(seed=1, n_clips=8, n_samples=480000).numpy()
        w = np.ones(6144, np.float32)
        t0 = time.perf_counter()
        n = sum(o.forward(xs[c], tb, rms_weight=w)[2].shape[0] for c in range(8))
        res["bursts_8x30s_tokens_per_s"] = n / (time.perf_counter() - t0)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs the dMel front end on one GPU only (asked for --gpus {args.gpus}); "
              "clips, streams and sequences are independent, so more GPUs would each take a share of the clips "
              "with no collective during the forward", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.steps is None:
        args.steps = {"batch": 20, "stream": 1000, "interleave": 5, "copy": 5, "shortconv": 20,
                      "shortconv_decode": 1000, "backward": 5, "hmlp": 10, "dft_gemm": 3,
                      "rounding": 1, "valu": 5}[args.workload]
    if args.workload == "stream":
        return bench_stream(args)
    if args.workload == "interleave":
        return bench_interleave(args)
    if args.workload == "copy":
        return bench_copy(args)
    if args.workload in ("shortconv", "shortconv_decode"):
        return bench_shortconv(args)
    if args.workload == "backward":
        return bench_backward(args)
    if args.workload == "hmlp":
        return bench_hmlp(args)
    if args.workload == "dft_gemm":
        return bench_dft_gemm(args)
    if args.workload == "rounding":
        return bench_rounding(args)
    if args.workload == "valu":
        return bench_valu(args)
    return bench_batch(args)


def bench_backward(args):
    """Backward of the front end's trainable parts on the 64 x 20 min batch,
    from a bf16 upstream gradient ~ N(0, 1e-3); the levels come from the front
    end before the timed region.  Two RMSNorm backwards are timed, then the
    table gradient (dmel_embed_backward, the token-order scatter):
    * from the sums the forward kept (dmel_embed_train writes them, then
      dmel_rms_backward_sums streams them): the training path, and the
      step the JSON line reports (rms from sums + table gradient);
    * dmel_rms_backward with the larger workspace (a first pass that
      recomputes the forward sum and keeps it, a second that streams it), for
      callers that do not keep the sums.
    The forward's extra cost of keeping the sums is timed as well
    (dmel_embed_train against dmel_embed, RMSNorm on, bf16 out)."""
    dev = "cuda"
    n_clips = args.clips
    clip_len = int(round(args.minutes * 60 * 16000))
    d = 6144
    audio = synth.speech_clips(seed=2, lengths=[clip_len] * n_clips, device=dev)
    ctx = dm.dmel_create(0)
    so, fo, T = dm.clip_offsets([clip_len] * n_clips, dev)
    lv = torch.empty((T, 80), dtype=torch.uint8, device=dev)
    dm.dmel_levels(ctx, audio, audio.numel(), so, fo, n_clips, T, None, lv)
    torch.cuda.synchronize()
    del audio
    table = synth.table_bf16(seed=1234).to(dev)
    w = torch.ones(d, dtype=torch.float32, device=dev)
    gram = torch.empty((1280, 1280), dtype=torch.float64, device=dev)
    dm.dmel_rms_gram(table, d, gram)
    scale = torch.empty(T, dtype=torch.float32, device=dev)
    dm.dmel_rms_scale(lv, T, gram, d, 1e-6, scale)
    dy = synth.activations_bf16(seed=21, n_tokens=T, channels=d, std=1e-3, device=dev)
    ds = torch.empty((T, d), dtype=torch.float32, device=dev)
    dw = torch.empty(d, dtype=torch.float32, device=dev)
    dt = torch.empty((1280, d), dtype=torch.float32, device=dev)
    sums = torch.empty((T, d), dtype=torch.float32, device=dev)
    y = torch.empty((T, d), dtype=torch.int16, device=dev)
    wb1 = dm.dmel_rms_backward_stored_workspace_bytes(T, d)   # keeps the sums between the two passes
    wb2 = dm.dmel_embed_backward_workspace_bytes(T, 80, 16, d)
    wb3 = dm.dmel_rms_backward_sums_workspace_bytes(T, d)
    ws = torch.empty(max(wb1, wb2, wb3), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def timed(calls, steps, warmup):
        """Mean event time of each call over `steps` rounds, and the wall time per round."""
        for _ in range(warmup):
            for c in calls:
                c()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for k in range(steps):
            events[k][0].record(stream)
            for i, c in enumerate(calls):
                c()
                events[k][i + 1].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(len(calls))] for e in events]).mean(axis=0)
        return per, wall

    fwd = lambda: dm.dmel_embed(lv, T, table, d, w, scale, y, dm.DMEL_BF16, d, None, stream)
    fwd_sums = lambda: dm.dmel_embed_train(lv, T, table, d, w, scale, y, dm.DMEL_BF16, d, None, sums, stream)
    rms_sums = lambda: dm.dmel_rms_backward_sums(sums, T, d, w, scale, dy, dm.DMEL_BF16, ds, dw, 0, ws, wb3, stream)
    rms_rec = lambda: dm.dmel_rms_backward(lv, T, 80, 16, table, d, w, scale, dy, dm.DMEL_BF16, ds, dw, 0, ws, wb1,
                                           stream)
    tab = lambda: dm.dmel_embed_backward(lv, T, 80, 16, ds, dm.DMEL_F32, d, dt, 0, ws, wb2, stream)
    (k_fwd, k_fwd_sums), _ = timed([fwd, fwd_sums], 3, 1)   # leaves the sums in place
    (k_rms_rec,), _ = timed([rms_rec], max(2, args.steps // 2), 1)
    (k_rms, k_tab), ms_step = timed([rms_sums, tab], args.steps, args.warmup)
    # the table gradient adds every token's gradient into one row per bin:
    # 80 x 6144 fp32 adds per token
    adds = 80 * d * T
    achieved = adds / (k_tab * 1e-3) / 1e12
    print(f"[bench] backward per step: rms from kept sums {k_rms:.3f} ms, table gradient {k_tab:.3f} ms; wall "
          f"{ms_step:.3f} ms; rms recomputing the sums {k_rms_rec:.3f} ms; forward embed {k_fwd:.3f} ms, "
          f"keeping the sums {k_fwd_sums:.3f} ms", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_backward(lv, table, dy, d)
    dm.dmel_destroy(ctx)
    line = {
        "metric": "backward tokens/s (RMSNorm + table gradient of the dMel embedding)",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"dMel backward: {n_clips} clips x {args.minutes:g} min ({T} tokens), table "
                               f"1280x6144, bf16 upstream gradient, RMSNorm backward from the sums the forward "
                               f"kept (dmel_embed_train: {k_fwd_sums - k_fwd:.2f} ms more than dmel_embed) + "
                               f"token-order table gradient",
                   "global_batch": n_clips, "seq_len": T // n_clips, "parallelism": "single GPU"},
        "kernel_ms": {"rms_backward_from_sums": float(k_rms), "table_gradient": float(k_tab),
                      "rms_backward_recomputing_sums": float(k_rms_rec), "embed_forward": float(k_fwd),
                      "embed_forward_keeping_sums": float(k_fwd_sums)},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_ADD_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_ADD_TFLOPS, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def bench_dft_gemm(args):
    """The two ways to the log-mel of the 64 x 20 min batch (1,536,000 frames):
    the mixed-radix FFT staged in LDS (dmel_frames) and the DFT as one bf16x3
    matrix-core product (dmel_bench_frames_dft_gemm of the benchmark-only
    library: split frames, GEMM over
    K = 4800 into 1792 fp32 columns, power + mel + log).  A step = one call of
    each, timed separately with HIP events.  `value` is the DFT-as-GEMM
    variant's frames/s; the FFT's is beside it."""
    dev = "cuda"
    n_clips = args.clips
    clip_len = int(round(args.minutes * 60 * 16000))
    audio = synth.speech_clips(seed=2, lengths=[clip_len] * n_clips, device=dev)
    ctx = dm.dmel_create(0)
    so, fo, T = dm.clip_offsets([clip_len] * n_clips, dev)
    lm_fft = torch.empty((T, 80), dtype=torch.float32, device=dev)
    lm_mm = torch.empty((T, 80), dtype=torch.float32, device=dev)
    from encoder_free_audio_amd import bench_ext as be
    mat = torch.empty(be.dmel_bench_dft_matrix_bytes(), dtype=torch.uint8, device=dev)
    wsb = be.dmel_bench_dft_gemm_workspace_bytes(T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    be.dmel_bench_dft_matrix(mat, stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dm.dmel_frames(ctx, audio, audio.numel(), so, fo, n_clips, T, None, lm_fft, stream)
        if ev is not None:
            ev[1].record(stream)
        be.dmel_bench_frames_dft_gemm(ctx, audio, audio.numel(), so, fo, n_clips, T, None, mat, lm_mm, ws, wsb,
                                      stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(2)] for e in events])
    ms_fft, ms_mm = per.mean(axis=0)
    a, b = np.clip(lm_fft.cpu().numpy(), -7, 2), np.clip(lm_mm.cpu().numpy(), -7, 2)
    diff = float(np.abs(a - b).max())
    flops_mm = 2.0 * 1792 * 4800 * T
    achieved = flops_mm / (ms_mm * 1e-3) / 1e12
    print(f"[bench] log-mel of {T} frames: LDS FFT {ms_fft:.3f} ms, DFT as GEMM {ms_mm:.3f} ms "
          f"({ms_mm / ms_fft:.1f}x); max |difference| of the clamped log-mel {diff:.2e}", file=sys.stderr, flush=True)
    dm.dmel_destroy(ctx)
    line = {
        "metric": "audio frames/s (log-mel of 16 kHz audio, DFT as a bf16x3 matrix-core product)",
        "value": T / (ms_mm * 1e-3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": float(ms_mm),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"log-mel of {n_clips} speech-like clips x {args.minutes:g} min ({T} frames): "
                               f"framing, 1600-point DFT as a [T, 4800] x [4800, 1792] bf16 product, power, "
                               f"80 mel filters, log",
                   "global_batch": n_clips, "seq_len": T // n_clips, "parallelism": "single GPU"},
        "kernel_ms": {"lds_fft_frames": float(ms_fft), "dft_gemm_frames": float(ms_mm)},
        "fft_frames_per_s": T / (ms_fft * 1e-3),
        "max_clamped_logmel_difference": diff,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_rounding(args):
    """In-bounds probe of how one add c + e (c fp32, e a bf16 value) rounds on
    this chip: by v_add_f32, by a matrix-core product with c as accumulator
    and a one-hot row selecting e, by the same product with a zero
    accumulator (e passed through), and by the bf16 dot instruction; each
    against the round-to-nearest-even sum numpy computes on the host.  The
    bag-of-bins embedding needs exactly that rounding for every add.  Cases:
    random pairs whose sum is inexact, exact midpoints (ties), and signed
    zeros.  Prints one JSON line of counts."""
    from encoder_free_audio_amd import bench_ext as be
    rng = np.random.default_rng(77)
    n = 1 << 24
    # c: sign, exponent in [-20, 20], random 23-bit mantissa
    c = (rng.choice([-1.0, 1.0], n) * np.ldexp(1.0 + rng.integers(0, 1 << 23, n) / float(1 << 23),
                                               rng.integers(-20, 21, n))).astype(np.float32)
    kind = np.zeros(n, np.int8)   # 0 random, 1 tie, 2 signed zero
    # random e: c scaled by 2^U[-12, 2], rounded to bf16 (varied alignment)
    e = (c.astype(np.float64) * np.ldexp(rng.uniform(0.5, 1.0, n), rng.integers(-12, 3, n))
         * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    # ties: e = (2k + 1) 2^(E - 24) lands c + e exactly between two fp32
    # values of c's binade (k < 64, so e has at most 7 significant bits)
    t = rng.random(n) < 0.25
    ex = np.frexp(c)[1] - 1
    k = rng.integers(0, 64, n)
    e_tie = (rng.choice([-1.0, 1.0], n) * np.ldexp(2.0 * k + 1.0, ex - 24)).astype(np.float32)
    e = np.where(t, e_tie, e)
    kind[t] = 1
    z = rng.random(n) < 0.01
    c = np.where(z, np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)), c).astype(np.float32)
    e = np.where(z, np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)), e).astype(np.float32)
    kind[z] = 2
    e_bits = (e.view(np.uint32) >> 16).astype(np.uint16)          # bf16 by truncation: exact for ties and zeros
    ef = (e_bits.astype(np.uint32) << 16).view(np.float32)
    want = (c + ef).astype(np.float32)                                # numpy: IEEE fp32 add, nearest even
    exact = c.astype(np.float64) + ef.astype(np.float64)              # exact: both fit in fp64's 53 bits
    inexact = exact != want.astype(np.float64)
    # a tie: the exact sum lies halfway between the nearest-even result and its other neighbour
    other = np.nextafter(want, np.where(exact > want, np.float32(np.inf), np.float32(-np.inf))).astype(np.float64)
    kind[(kind == 1) & ~(inexact & (np.abs(exact - want) == np.abs(exact - other)))] = 0
    cd = torch.from_numpy(c).cuda()
    ed = torch.from_numpy(e_bits.view(np.int16)).cuda()
    out = torch.empty((4, n), dtype=torch.float32, device="cuda")
    be.dmel_bench_rounding_probe(cd, ed, n, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    wb = want.view(np.uint32)
    res = {"workload": "rounding_probe", "cases": n, "random_cases": int((kind == 0).sum()),
           "tie_cases": int((kind == 1).sum()), "zero_cases": int((kind == 2).sum()),
           "inexact_cases": int(inexact.sum())}
    for i, name in ((0, "v_add_f32"), (1, "mfma_accumulate"), (3, "dot2_bf16")):
        bad = got[i].view(np.uint32) != wb
        res[name] = {"mismatches": int(bad.sum()), "mismatches_inexact": int((bad & inexact).sum()),
                     "mismatches_ties": int((bad & (kind == 1)).sum()), "mismatches_zeros": int((bad & (kind == 2)).sum()),
                     "below_nearest_even": int((bad & (got[i].astype(np.float64) < want)).sum())}
    bad = got[2].view(np.uint32) != ef.view(np.uint32)
    res["mfma_zero_accumulator_vs_e"] = {"mismatches": int(bad.sum()),
                                         "mismatches_nonzero_e": int((bad & (ef != 0)).sum()),
                                         "mismatches_negative_zero_e": int((bad & (e_bits == 0x8000)).sum())}
    print(json.dumps(res), flush=True)


def bench_hmlp(args):
    """hMLP image front end: 32 bf16 images of 1280 x 1280 (32768 patches),
    widths 1536, 1536, 1536, 6144, bf16 out.  One step = dmel_hmlp_forward.
    The stage-2 GEMM (the dominant launch: 302 MFLOP per patch) is also timed
    alone through dmel_hmlp_stage for the roofline."""
    dev = "cuda"
    n, H, W, hidden, d = 32, 1280, 1280, 1536, 6144
    P = n * (H // 40) * (W // 40)
    images = synth.table_bf16(seed=5, rows=n * H * W, d_model=3, std=1.0, device=dev)
    rng = np.random.default_rng(6)
    shapes = [(hidden, 75), (hidden, 4 * hidden), (hidden, 4 * hidden), (d, 4 * hidden)]
    ws = []
    for nn_, k in shapes:
        ws.append(synth.table_bf16(seed=int(rng.integers(1 << 30)), rows=nn_, d_model=k, std=1.0 / np.sqrt(k)).to(dev))
        ws.append(torch.from_numpy((rng.standard_normal(nn_) * 0.1).astype(np.float32)).to(dev))
    out = torch.empty((P, d), dtype=torch.int16, device=dev)
    wsb = dm.dmel_hmlp_workspace_bytes(n, H, W, hidden)
    wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        dm.dmel_hmlp_forward(images, n, H, W, *ws, hidden, d, out, dm.DMEL_BF16, wsp, wsb, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    # stage 2 alone (same kernel, same shape as inside the forward)
    x2 = torch.empty((P * 16, 4 * hidden), dtype=torch.int16, device=dev)
    x2.view(torch.bfloat16).normal_()
    y2 = torch.empty((P * 16, hidden), dtype=torch.int16, device=dev)
    for _ in range(2):
        dm.dmel_hmlp_stage(x2, P * 16, 4 * hidden, ws[2], ws[3], hidden, 1, y2, dm.DMEL_BF16, stream)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(5):
        dm.dmel_hmlp_stage(x2, P * 16, 4 * hidden, ws[2], ws[3], hidden, 1, y2, dm.DMEL_BF16, stream)
    f1.record(stream)
    torch.cuda.synchronize()
    k2 = f0.elapsed_time(f1) / 5
    flops2 = 2.0 * P * 16 * (4 * hidden) * hidden
    achieved = flops2 / (k2 * 1e-3) / 1e12
    flops_all = 2.0 * P * (64 * 75 * hidden + 16 * 4 * hidden * hidden + 4 * 4 * hidden * hidden + 4 * hidden * d)
    print(f"[bench] hmlp step {ms_ev:.3f} ms (events), wall {ms_step:.3f} ms; stage-2 GEMM {k2:.3f} ms "
          f"= {achieved:.0f} TFLOP/s; whole stem {flops_all / (ms_ev * 1e-3) / 1e12:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_hmlp(images, ws, H, W)
    line = {
        "metric": "image patches/s (hMLP front end, 40 x 40 patches -> 6144-d)",
        "value": P / (ms_step * 1e-3),
        "unit": "patches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"hMLP stem: {n} images x {H} x {W} ({P} patches), widths {hidden}/{hidden}/{hidden}/"
                               f"{d}, bf16 matrix-core products, fp32 accumulation, bf16 out",
                   "global_batch": n, "seq_len": P // n, "parallelism": "single GPU"},
        "kernel_ms": {"forward": ms_ev, "stage2_gemm": k2},
        "tflops_stem": flops_all / (ms_ev * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_hmlp(images, ws, H, W):
    """The hMLP oracle (fp64) on a bounded sample: the first 8 patches of the
    first image, one process."""
    from oracle import hmlp_oracle as ho  # noqa: E402  (test infrastructure)

    img = images[: H * W].view(1, H, W, 3)[:, :40, :320, :].contiguous().cpu().numpy().view(np.uint16)
    wn = [(ws[2 * i].cpu().numpy().view(np.uint16), ws[2 * i + 1].cpu().numpy()) for i in range(4)]
    t0 = time.perf_counter()
    ho.hmlp(img, wn)
    dt = time.perf_counter() - t0
    return {"value": 8 / dt, "unit": "patches/s", "cores": 1, "kind": "oracle",
            "sample": f"8 patches (a 40 x 320 strip of the first image), full widths, one process, {dt:.1f} s wall"}


def cpu_baseline_backward(lv, table, dy, d):
    """The oracle's backward (fp64 RMSNorm backward, fixed-order fp32 table
    gradient) on a bounded sample: the first 3000 tokens, one process."""
    from oracle import dmel_oracle as o  # noqa: E402  (test infrastructure)

    n = 3000
    lvs = lv[:n].cpu().numpy()
    tb = table.cpu().numpy().view(np.uint16)
    dys = o.bf16_to_f32(dy[:n].cpu().numpy().view(np.uint16))
    t0 = time.perf_counter()
    ds, _, _, _ = o.rms_backward(lvs, tb, np.ones(d, np.float32), dys)
    o.embed_backward(lvs, ds.astype(np.float32))
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens of the batch, RMSNorm backward + table gradient, one process, "
                      f"{dt:.1f} s wall"}


def cpu_baseline_shortconv(x, w, st, S, L, decode):
    """The short-convolution oracle (fp64, one process) on a bounded sample of
    the same workload (about 10 s of CPU work): 8 requests x 8000 tokens of the
    prefill, or up to 8000 decode steps of 8 requests."""
    from oracle import shortconv_oracle as sc  # noqa: E402  (test infrastructure)

    C = x.shape[1]
    n_req, n_tok = 8, 8000
    if decode:
        n_tok = min(n_tok, x.shape[0] // S)
        xs = x[: n_tok * S].view(n_tok, S, C)[:, :n_req].permute(1, 0, 2).reshape(n_req * n_tok, C)
    else:
        xs = x.view(S, L, C)[:n_req, :n_tok].reshape(n_req * n_tok, C)
    xb = xs.cpu().numpy().view(np.uint16)
    stb = st[:n_req].cpu().numpy().view(np.uint16)
    wn = w.cpu().numpy().astype(np.float64)
    off = np.arange(0, n_req * n_tok + 1, n_tok)
    t0 = time.perf_counter()
    sc.shortconv(xb, off, wn, stb)
    dt = time.perf_counter() - t0
    return {"value": n_req * n_tok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_req} requests x {n_tok} tokens x {C} channels ({'decode steps' if decode else 'prefill'}), "
                      f"state in and out, one process, {dt:.1f} s wall"}


def bench_shortconv(args):
    """The decoder's short convolution (width 4, per-request state): prefill of
    64 requests x 24,000 tokens x 6144 channels, or decode steps of one token
    for each of 4096 requests with the state carried in two buffers.  Inputs
    bf16 ~ N(0, 1), taps ~ U(-0.5, 0.5), bf16 output."""
    dev = "cuda"
    C = 6144
    decode = args.workload == "shortconv_decode"
    S, L = (args.streams, 1) if decode else (64, 24000)
    T = S * L
    n_x = T if not decode else T * args.steps
    x = synth.activations_bf16(seed=90, n_tokens=n_x, channels=C, device=dev)
    w = synth.shortconv_weight(seed=91, channels=C).to(dev)
    st = [synth.activations_bf16(seed=92, n_tokens=S * 3, channels=C, device=dev).view(S, 3, C),
          torch.empty((S, 3, C), dtype=torch.int16, device=dev)]
    off = torch.arange(0, T + 1, L, dtype=torch.int64, device=dev)
    y = torch.empty((T, C), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    def step(k, ev=None):
        xk = x[(k % (n_x // T)) * T: (k % (n_x // T) + 1) * T]
        if ev is not None:
            ev[0].record(stream)
        dm.dmel_shortconv(xk, T, C, off, S, w, st[k % 2], st[(k + 1) % 2], y, dm.DMEL_BF16, stream)
        if ev is not None:
            ev[1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(k, events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = np.array([e[0].elapsed_time(e[1]) for e in events])
    k_ms = float(per.mean())
    ms_step = wall * 1e3 / args.steps
    bytes_launch = T * C * 2 * 2 + S * 3 * C * 2 * 2 + C * 16 + (S + 1) * 8
    achieved = bytes_launch / (k_ms * 1e-3) / 1e9
    line = {
        "metric": "short-convolution tokens/s (width 4, 6144 channels, per-request state)",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (f"shortconv decode: {S} requests x 1 token per step, state carried" if decode else
                                f"shortconv prefill: {S} requests x {L} tokens") + f", {C} channels, bf16 in/out",
                   "global_batch": S, "seq_len": L, "parallelism": "single GPU"},
        "kernel_ms": {"shortconv": k_ms, "p50": float(np.percentile(per, 50)), "p99": float(np.percentile(per, 99))},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_shortconv(x, w, st[0], S, L, decode),
    }
    print(f"[bench] shortconv kernel {k_ms:.4f} ms per launch ({bytes_launch / 1e9:.3f} GB algorithmic), "
          f"wall {ms_step:.4f} ms per step", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


def bench_copy(args):
    """A plain device-to-device copy of 1 GiB: its FETCH_SIZE / WRITE_SIZE
    counter values, against the 1 GiB it reads and writes, scale the counter
    readings of the front-end kernels to bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(json.dumps({"workload": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "ms_per_copy": ms,
                      "GBps": 8 * n / (ms * 1e-3) / 1e9}), flush=True)


VALU_KINDS = ("v_add_f32 VOP2, VGPR operands", "v_add_f32 VOP3, VGPR operands", "v_add_f32 with an SGPR operand",
              "v_fmac_f32 VOP2", "v_fma_f32 VOP3", "v_mul_f32 VOP2", "v_lshlrev_b32 by 16",
              "v_and_b32 with a VGPR mask", "v_and_b32 with a literal mask", "v_cvt_f32_bf16 SDWA high half",
              "v_cvt_f32_bf16 VOP1", "v_mov_b32 SDWA low word to high word", "v_perm_b32",
              "v_alignbit_b32 by 16", "v_mul_u32_u24 by 65536")
LDS_MODES = ("linear", "one address", "16-float rows, 80 B pitch", "16-float rows, 64 B pitch")


def bench_valu(args):
    """Issue rate of single vector-ALU instruction forms over the whole chip
    (dmel_bench_valu_rate: 16 independent register chains per lane, no memory
    in the loop).  8192 workgroups of 256 lanes (32 waves per CU) x 4096
    rounds x 16 chains = 1.37e11 lane-operations per launch (about 2 ms);
    the rate is lane-operations per second, timed with HIP events per
    launch.  Then v_add_f32 at 1, 2, 4 and 8 waves per SIMD (same lane-
    operations), and the LDS read rate of dmel_bench_lds_rate for its four
    access patterns (4096 workgroups of 256 lanes x 2048 rounds x 64 B)."""
    from encoder_free_audio_amd import bench_ext as be
    blocks, iters = 8192, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ops = float(blocks) * 256 * iters * 16
    rates = {}
    kinds = list(enumerate(VALU_KINDS)) + [(15, "mfma_32x32x16_bf16 only"), (16, "mfma_32x32x16_bf16 + 16 v_add_f32")]
    for kind, name in kinds:
        for _ in range(args.warmup):
            be.dmel_bench_valu_rate(kind, blocks, iters, out, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for k in range(args.steps):
            be.dmel_bench_valu_rate(kind, blocks, iters, out, stream)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
        ms_mean = float(np.mean(ms))
        if kind >= 15:
            # rounds per SIMD: 8192 x 4 waves over 1024 SIMDs, `iters` rounds each
            clk = ms_mean * 1e-3 * 2.4e9 / (blocks * 4 / 1024 * iters)
            rates[name] = {"ms_per_launch": ms_mean, "clk_per_round_per_SIMD_at_2.4GHz": clk}
            print(f"[bench] {name}: {ms_mean:.3f} ms, {clk:.1f} clk per round per SIMD", file=sys.stderr, flush=True)
            continue
        rates[name] = {"ms_per_launch": ms_mean, "T_ops_per_s": ops / (ms_mean * 1e-3) / 1e12}
        print(f"[bench] {name}: {ms_mean:.3f} ms, {rates[name]['T_ops_per_s']:.1f} T lane-ops/s",
              file=sys.stderr, flush=True)
    # plain adds at lower occupancy: 256-lane workgroups are 4 waves, one per SIMD
    occ = {}
    for wps in (1, 2, 4, 8):
        b = 256 * wps
        it = iters * 32 // wps // 4
        for _ in range(args.warmup):
            be.dmel_bench_valu_rate(0, b, it, out, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            be.dmel_bench_valu_rate(0, b, it, out, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_mean = e0.elapsed_time(e1) / args.steps
        occ[f"{wps} waves per SIMD"] = {"ms_per_launch": ms_mean,
                                        "T_ops_per_s": float(b) * 256 * it * 16 / (ms_mean * 1e-3) / 1e12}
        print(f"[bench] v_add_f32 VOP2 at {wps} waves per SIMD: {occ[f'{wps} waves per SIMD']['T_ops_per_s']:.1f} "
              f"T lane-ops/s", file=sys.stderr, flush=True)
    # LDS: 4096 workgroups (four resident per CU) x 256 lanes x 2048 rounds x 64 B
    lblocks, liters = 4096, 2048
    lout = torch.empty(lblocks * 256, dtype=torch.float32, device="cuda")
    lbytes = float(lblocks) * 256 * liters * 64
    lds = {}
    for mode, name in enumerate(LDS_MODES):
        for _ in range(args.warmup):
            be.dmel_bench_lds_rate(mode, lblocks, liters, lout, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for k in range(args.steps):
            be.dmel_bench_lds_rate(mode, lblocks, liters, lout, stream)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        ms_mean = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]))
        tbps = lbytes / (ms_mean * 1e-3) / 1e12
        lds[name] = {"ms_per_launch": ms_mean, "TB_per_s": tbps, "B_per_clk_per_CU_at_2.4GHz": tbps * 1e12 / 256 / 2.4e9}
        print(f"[bench] LDS ds_read_b128, {name}: {ms_mean:.3f} ms, {tbps:.1f} TB/s", file=sys.stderr, flush=True)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lout).all())
    print(json.dumps({"workload": "valu_issue_rates", "blocks": blocks, "threads": 256, "rounds": iters,
                      "chains": 16, "lane_ops_per_launch": ops, "rates": rates,
                      "clock_x_lanes_T": 256 * 64 * 2.4e9 / 1e12, "datasheet_fp32_vector_T": PEAK_FP32_TFLOPS,
                      "v_add_f32_by_occupancy": occ,
                      "lds_read": {"blocks": lblocks, "threads": 256, "rounds": liters,
                                   "bytes_per_launch": lbytes, "modes": lds}}),
          flush=True)


def _base_line(args, value, ms_step, workload, extra):
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": {"workload": workload},
    }
    line.update(extra)
    return line


def bench_stream(args):
    """Streaming: every step each of S streams delivers one new 800-sample hop;
    dmel_forward turns the S hops (with each stream's previous hop as carry)
    into S tokens.  Reports per-step latency percentiles and tokens/s."""
    dev = "cuda"
    S = args.streams
    K = args.steps
    print(f"[bench] generating {S} streams x {K} hops on the GPU", file=sys.stderr, flush=True)
    hops = synth.streaming_hops(seed=3, n_streams=S, n_steps=K + args.warmup, device=dev)
    table = synth.table_bf16(seed=1234).to(dev)
    rms_w = torch.ones(6144, dtype=torch.float32, device=dev)
    gram = torch.empty((1280, 1280), dtype=torch.float64, device=dev)
    ctx = dm.dmel_create(0)
    dm.dmel_rms_gram(table, 6144, gram)
    so, fo, _ = dm.clip_offsets([800] * S, dev)
    ws = torch.empty(dm.dmel_forward_workspace_bytes(S), dtype=torch.uint8, device=dev)
    out = torch.empty((S, 6144), dtype=torch.int16, device=dev)
    zeros = torch.zeros((S, 800), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(k):
        carry = zeros if k == 0 else hops[k - 1]
        dm.dmel_forward(ctx, hops[k], S * 800, so, fo, S, S, carry, table, 6144, rms_w, gram, 1e-6, out,
                        dm.DMEL_BF16, 6144, None, ws, ws.numel(), stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(K):
        step(args.warmup + k)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(K)])
    dm.dmel_destroy(ctx)
    line = _base_line(args, S * K / wall, wall * 1e3 / K,
                      f"dMel streaming: {S} streams, one 800-sample hop per stream per step with an 800-sample "
                      f"carry, {K} steps, RMSNorm on, bf16 out",
                      {"p50_step_ms": float(np.percentile(per, 50)), "p99_step_ms": float(np.percentile(per, 99)),
                       "steps": K})
    line["config"].update({"streams": S, "parallelism": "single GPU"})
    print(json.dumps(line), flush=True)


def bench_interleave(args):
    """Interleaved sequences: 256 x 32768 positions, 40% audio frames (dmel_forward
    with out_rows) and 60% text rows (dmel_gather_rows) written into one bf16
    [256, 32768, 6144] output.  One step = both calls for the whole batch."""
    dev = "cuda"
    lay = synth.interleave_layout(seed=4)
    n_seq, L = lay["n_seq"], lay["seq_len"]
    kind, seq, start, ln = lay["seg_kind"], lay["seg_seq"], lay["seg_start"], lay["seg_len"]
    a_idx = np.nonzero(kind == 1)[0]
    t_idx = np.nonzero(kind == 0)[0]
    clip_frames = ln[a_idx]
    print(f"[bench] generating {clip_frames.sum()} audio frames and the 131072-row text table", file=sys.stderr,
          flush=True)
    audio = synth.speech_clips(seed=4, lengths=(clip_frames * 800).tolist(), device=dev)
    table = synth.table_bf16(seed=1234).to(dev)
    text = synth.table_bf16(seed=1235, rows=131072, d_model=6144, device=dev)
    a_rows = torch.from_numpy(np.concatenate([seq[i] * L + start[i] + np.arange(ln[i]) for i in a_idx])).to(dev)
    t_pos = np.concatenate([seq[i] * L + start[i] + np.arange(ln[i]) for i in t_idx])
    t_rows = torch.from_numpy(t_pos).to(dev)
    ids = torch.from_numpy(lay["ids"].reshape(-1)[t_pos].astype(np.int32)).to(dev)
    out = torch.empty((n_seq * L, 6144), dtype=torch.int16, device=dev)
    ctx = dm.dmel_create(0)
    so, fo, T = dm.clip_offsets((clip_frames * 800).tolist(), dev)
    ws = torch.empty(dm.dmel_forward_workspace_bytes(T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    n_text = t_pos.size

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dm.dmel_forward(ctx, audio, audio.numel(), so, fo, len(a_idx), T, None, table, 6144, None, None, 1e-6,
                        out, dm.DMEL_BF16, 6144, a_rows, ws, ws.numel(), stream)
        if ev is not None:
            ev[1].record(stream)
        dm.dmel_gather_rows(text, 131072, 6144, ids, n_text, out, 6144, t_rows, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in evs]).mean(axis=0)
    dm.dmel_destroy(ctx)
    ms = wall * 1e3 / args.steps
    gather_bytes = n_text * 6144 * 2 * 2
    line = _base_line(args, T / (ms * 1e-3), ms,
                      f"dMel interleave: {n_seq} x {L} positions, {T} audio frames in {len(a_idx)} clips + "
                      f"{n_text} text rows of a 131072x6144 bf16 table, one bf16 output, RMSNorm off",
                      {"positions_per_s": n_seq * L / (ms * 1e-3),
                       "kernel_ms": {"audio_forward": float(per[0]), "text_gather": float(per[1])},
                       "text_gather_GBps": gather_bytes / (per[1] * 1e-3) / 1e9})
    line["config"].update({"sequences": n_seq, "seq_len": L, "parallelism": "single GPU"})
    print(json.dumps(line), flush=True)


def bench_batch(args):
    dev = "cuda"
    n_clips = args.clips
    clip_len = int(round(args.minutes * 60 * 16000))
    T_clip = dm.dmel_num_frames(clip_len)
    n_tok = n_clips * T_clip
    d = 6144
    cfg = args.config or dm.dmel_default_config()
    n_bins, n_lv = cfg["n_mel_bins"], cfg["mel_vocab_size"]
    released = cfg == dm.dmel_default_config()
    lay = dict(n_bins=n_bins, n_levels=n_lv)
    print(f"[bench] generating {n_clips} x {args.minutes:g} min speech-like audio on the GPU", file=sys.stderr,
          flush=True)
    t0 = time.time()
    audio = synth.speech_clips(seed=2, lengths=[clip_len] * n_clips, device=dev)
    table = synth.table_bf16(seed=1234, rows=n_bins * n_lv).to(dev)
    rms_w = torch.ones(d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    ctx = dm.dmel_create_config(0, cfg)
    so, fo, T = dm.clip_offsets([clip_len] * n_clips, dev)
    assert T == n_tok
    out = torch.empty((n_tok, d), dtype=torch.int16, device=dev)
    gram = torch.empty((1280, 1280), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    # the Gram matrix of the table: once per table (weight preparation), outside the step
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    dm.dmel_rms_gram(table, d, gram, stream, **lay)
    g1.record(stream)
    ws = torch.empty(dm.dmel_forward_workspace_bytes(n_tok), dtype=torch.uint8, device=dev)

    def step():
        dm.dmel_forward(ctx, audio, audio.numel(), so, fo, n_clips, n_tok, None, table, d, rms_w, gram, 1e-6, out,
                        dm.DMEL_BF16, d, None, ws, ws.numel(), stream)

    # timed region: the product call, one dmel_forward per step
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev[0].record(stream)
    for k in range(args.steps):
        step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)])
    ms_step = wall * 1e3 / args.steps
    tok_s = n_tok / (ms_step * 1e-3)
    gram_ms = g0.elapsed_time(g1)

    # per-kernel split: the same three launches dmel_forward enqueues, called
    # one by one with events between them (same kernels, same sizes)
    levels = ws[: n_tok * n_bins].view(n_tok, n_bins)
    scale = torch.empty(n_tok, dtype=torch.float32, device=dev)

    def split(e=None):
        if e is not None:
            e[0].record(stream)
        dm.dmel_levels(ctx, audio, audio.numel(), so, fo, n_clips, n_tok, None, levels, stream)
        if e is not None:
            e[1].record(stream)
        dm.dmel_rms_scale(levels, n_tok, gram, d, 1e-6, scale, stream, **lay)
        if e is not None:
            e[2].record(stream)
        dm.dmel_embed(levels, n_tok, table, d, rms_w, scale, out, dm.DMEL_BF16, d, None, stream, **lay)
        if e is not None:
            e[3].record(stream)

    split()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        split(events[k])
    torch.cuda.synchronize()
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in events])  # ms
    k_front, k_scale, k_embed = per.mean(axis=0)
    embed_adds = (n_bins - 1) * d * n_tok   # 79 x 6144 per token for the released 80 bins
    achieved = embed_adds / (k_embed * 1e-3) / 1e12
    hbm = HBM_BYTES_PER_TOKEN * n_tok / (ms_step * 1e-3) / 1e9
    print(f"[bench] dmel_forward {ms_step:.3f} ms per step (events: p50 {np.median(step_ms):.3f}, max "
          f"{step_ms.max():.3f}); split: levels {k_front:.3f} ms, rms_scale {k_scale:.3f} ms, embed {k_embed:.3f} ms; "
          f"Gram (once per table) {gram_ms:.3f} ms", file=sys.stderr, flush=True)

    # a plain 1 GiB device copy, timed after the steps: the HBM rate this box
    # reaches, to set the step's algorithmic rate against
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * 4 * (1 << 28) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    front_tflops = FRONT_FLOPS_PER_FRAME * n_tok / (k_front * 1e-3) / 1e12

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        # the GPU's results for the oracle's sample: the product call's tokens,
        # its levels, and the log-mel of the same frames (dmel_frames)
        step()
        lm = torch.empty((n_tok, n_bins), dtype=torch.float32, device=dev)
        dm.dmel_frames(ctx, audio, audio.numel(), so, fo, n_clips, n_tok, None, lm, stream)
        torch.cuda.synchronize()

        def gpu_sample(c, f):
            r = slice(c * T_clip, c * T_clip + f)
            return (lm[r].cpu().numpy(), ws[: n_tok * n_bins].view(n_tok, n_bins)[r].cpu().numpy(),
                    out[r].cpu().numpy().view(np.uint16))
        try:
            cpu, parity = cpu_baseline(audio, clip_len, table, n_clips, args.cpu_frames, gpu_sample,
                                       None if released else cfg)
            if released:
                cpu["one_core"] = one_core_baseline()
        except Exception as e:  # report, never hide the GPU line
            cpu = {"value": None, "unit": "tokens/s", "cores": 0, "kind": "oracle", "sample": f"failed: {e}"}
    dm.dmel_destroy(ctx)
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"dMel forward (dmel_forward per step): {n_clips} clips x {args.minutes:g} min of "
                               f"16 kHz speech-like audio ({n_tok} tokens), {n_bins} mel bins x {n_lv} levels over "
                               f"[{cfg['min_value']:g}, {cfg['max_value']:g}], table {n_bins * n_lv}x6144 bf16, "
                               f"fp32 sum, RMSNorm on, bf16 out; the table's Gram matrix is computed once per table "
                               f"({gram_ms:.2f} ms), outside the step",
                   "global_batch": n_clips, "seq_len": T_clip, "parallelism": "single GPU"},
        "hbm_achieved_GBps": hbm,
        "hbm_frac": hbm / PEAK_HBM_GBPS,
        "copy_GBps": copy_gbps,
        "hbm_frac_of_copy": hbm / copy_gbps,
        "embed_lds_gather": {"bytes_per_add": 4, "achieved_TBps": achieved * 4, "ceiling_TBps": LDS_GATHER_TBPS,
                             "frac": achieved * 4 / LDS_GATHER_TBPS},
        "frontend_TFLOPs": front_tflops,
        "frontend_frac_of_fp32_peak": front_tflops / PEAK_FP32_TFLOPS,
        "step_ms_p50": float(np.median(step_ms)),
        "kernel_ms": {"frontend_levels": k_front, "rms_scale": k_scale, "embed": k_embed, "gram_once": gram_ms},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_ADD_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_ADD_TFLOPS,
                     "traffic": embed_traffic() if (n_clips, clip_len) == (64, 19_200_000) and released else None},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
