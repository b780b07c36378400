"""Oracle work for the full-size GPU parity tests, spread over host processes.

The test copies the GPU's inputs and results to host memory, stores them in
``DATA`` and forks the pool, so the workers read them without copies.  Each
job runs the CPU oracle on one clip and compares the GPU's results with it to
the bars of ``tests/_parity.py``; a failed bar raises in the worker and the
pool re-raises it in the test.  Nothing here touches the GPU."""

from __future__ import annotations

import numpy as np

DATA: dict = {}


def pool_size(n_jobs: int) -> int:
    import os
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(cores, 16, n_jobs))


def clip_job(c: int) -> dict:
    """Log-mel and levels of every frame of clip c (DATA["clips"][c]: its
    audio, the GPU's levels and, if present, log-mel and tokens); with tokens,
    every token whose levels match the oracle's is compared too."""
    from threadpoolctl import threadpool_limits

    from oracle import dmel_oracle as o
    from tests import _parity as P

    clip = DATA["clips"][c]
    with threadpool_limits(1):
        lm_o = o.log_mel(clip["audio"])
        lv_o = o.quantize(lm_o)
        lm_g = clip.get("logmel")
        lv_g = clip["levels"]
        res = {"frames": int(lv_g.shape[0])}
        if lm_g is not None:
            err_c, err_u = P.check_logmel(lm_g, lm_o)
            res.update(max_err_clamped=err_c, max_err_unclamped=err_u)
        band, forgiven, frames = P.check_levels(lv_g, lm_o, lv_o, gpu_lm=lm_g)
        res.update(edge_band=band, forgiven=forgiven, frames_affected=frames)
        tok = clip.get("tokens")
        if tok is not None:
            same = np.all(lv_g == lv_o, axis=1)
            w = DATA.get("rms_weight")
            want, exact = o.embed(lv_o[same], DATA["table"], rms_weight=w)
            got = tok[same]
            if w is None:
                assert np.array_equal(got, want), "tokens differ from the oracle"
                ulp1 = 0
            else:
                ulp1 = P.check_rms_bf16(got, exact)
            res.update(tokens_checked=int(same.sum()), tokens_bit_exact=int(np.all(got == want, axis=1).sum()),
                       bf16_midpoint_ulps=ulp1)
    return res


def merge(results) -> dict:
    out = {}
    for r in results:
        for k, v in r.items():
            if k.startswith("max_"):
                out[k] = max(out.get(k, 0.0), v)
            else:
                out[k] = out.get(k, 0) + v
    return out


def run() -> dict:
    """Every clip of DATA["clips"] on a pool of forked host processes."""
    import multiprocessing as mp
    jobs = list(range(len(DATA["clips"])))
    ctx = mp.get_context("fork")
    with ctx.Pool(pool_size(len(jobs))) as pool:
        return merge(pool.map(clip_job, jobs, chunksize=1))
