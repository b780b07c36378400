"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, reports the method's constants, and rejects bad arguments in host
code before any HIP call (no GPU needed for any of these)."""

import os
import re
import subprocess
import sys

import pytest

from oracle import dmel_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dm():
    from encoder_free_audio_amd import dmel
    dmel.lib()
    return dmel


def _header_symbols():
    with open(os.path.join(ROOT, "include", "dmel.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmel_[a-z_]+)\s*\(", text)))


def test_exports_every_header_symbol(dm):
    syms = _header_symbols()
    assert len(syms) >= 16
    assert sorted(dm.EXPORTS) == syms
    out = subprocess.run(["nm", "-D", "--defined-only", dm.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dmel_\w+)", out))
    missing = [s for s in syms if s not in exported]
    assert not missing, missing


def test_params_match_the_method(dm):
    p = dm.dmel_get_params()
    assert p["sample_rate"] == o.SAMPLE_RATE and p["hop"] == o.HOP and p["window"] == o.WINDOW
    assert p["n_fft"] == o.N_FFT and p["n_bins"] == o.N_BINS
    assert p["n_mels"] == o.N_MELS and p["n_levels"] == o.N_LEVELS and p["n_rows"] == o.N_ROWS
    assert p["clamp_min"] == o.CLAMP_MIN and p["clamp_max"] == o.CLAMP_MAX
    assert abs(p["log_floor"] - o.LOG_FLOOR) < 1e-17
    assert p["f_min_hz"] == o.F_MIN and p["f_max_hz"] == o.F_MAX


def test_default_config_is_the_released_one(dm):
    c = dm.dmel_default_config()
    cfg = o.Config()
    assert c == {"n_mel_bins": cfg.n_mel_bins, "mel_vocab_size": cfg.mel_vocab_size,
                 "min_value": cfg.min_value, "max_value": cfg.max_value}


def test_config_validation(dm):
    # rejected in host code before any HIP call
    E = dm.DmelError
    good = dict(n_mel_bins=80, mel_vocab_size=16, min_value=-1.5, max_value=2.0)
    bad = [dict(n_mel_bins=0), dict(n_mel_bins=129), dict(mel_vocab_size=0), dict(mel_vocab_size=257),
           dict(min_value=2.0), dict(min_value=3.0), dict(min_value=float("nan")), dict(max_value=float("inf")),
           dict(min_value=1.0, max_value=1.0 + 2.0 ** -23)]
    for kw in bad:
        c = dict(good)
        c.update(kw)
        with pytest.raises(E) as e:
            dm.dmel_create_config(0, c)
        assert _code(e) == -1, (kw, str(e.value))
    with pytest.raises(E) as e:
        dm.dmel_get_config(None)
    assert _code(e) == -1


def test_num_frames(dm):
    for n in (0, 1, 799, 800, 801, 1599, 1600, 16000, 19_200_000, 2 ** 40 + 5):
        assert dm.dmel_num_frames(n) == o.num_frames(n)
    assert dm.dmel_num_frames(-1) == -1


def test_workspace_bytes(dm):
    assert dm.dmel_forward_workspace_bytes(0) == 0
    assert dm.dmel_forward_workspace_bytes(-5) == 0
    n = 1000
    b = dm.dmel_forward_workspace_bytes(n)
    assert b >= n * 80 + n * 4 and b % 256 == 0


FAKE = 1 << 20  # an aligned, never-dereferenced address: validation fails first


def _code(exc):
    return exc.value.code


def test_validation_frames(dm):
    E = dm.DmelError
    # negative counts
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, -1, FAKE, FAKE, 1, 0, None, FAKE)
    assert _code(e) == -1
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE, FAKE, -1, 0, None, FAKE)
    assert _code(e) == -1
    # more frames than the audio can hold
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE, FAKE, 1, 3, None, FAKE)
    assert _code(e) == -2
    # frames without clips
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE, FAKE, 0, 1, None, FAKE)
    assert _code(e) == -2
    # null output / audio
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE, FAKE, 1, 2, None, None)
    assert _code(e) == -1
    with pytest.raises(E) as e:
        dm.dmel_levels(None, None, 1600, FAKE, FAKE, 1, 2, None, FAKE)
    assert _code(e) == -1
    # misaligned audio / offsets
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE + 2, 1600, FAKE, FAKE, 1, 2, None, FAKE)
    assert _code(e) == -4
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE + 4, FAKE, 1, 2, None, FAKE)
    assert _code(e) == -4
    # everything else valid: a NULL context is reported last
    with pytest.raises(E) as e:
        dm.dmel_frames(None, FAKE, 1600, FAKE, FAKE, 1, 2, None, FAKE)
    assert _code(e) == -1 and "ctx" in str(e.value)
    assert "ctx" in dm.dmel_last_error()


def test_validation_embed(dm):
    E = dm.DmelError
    ok = dict(levels=FAKE, n_tokens=10, table=FAKE, d_model=6144, rms_weight=None, rms_scale=None, out=FAKE,
              out_dtype=0, out_row_stride=6144)

    ok.update(n_bins=80, n_levels=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        dm.dmel_embed(a["levels"], a["n_tokens"], a["table"], a["d_model"], a["rms_weight"], a["rms_scale"],
                      a["out"], a["out_dtype"], a["out_row_stride"], n_bins=a["n_bins"], n_levels=a["n_levels"])

    cases = [
        (dict(n_bins=0), -2),
        (dict(n_bins=81), -2),
        (dict(n_levels=0), -2),
        (dict(n_levels=17), -2),
        (dict(n_tokens=-1), -1),
        (dict(d_model=100), -2),
        (dict(d_model=0), -2),
        (dict(d_model=65536 + 16), -2),
        (dict(table=None), -1),
        (dict(table=FAKE + 8), -4),
        (dict(out_dtype=7), -3),
        (dict(out=None), -1),
        (dict(out=FAKE + 4), -4),
        (dict(out_row_stride=100), -2),
        (dict(out_row_stride=6148), -4),   # 12296 bytes: not a multiple of 16
        (dict(rms_weight=FAKE), -1),       # weight without scale
        (dict(levels=None), -1),
        (dict(levels=FAKE + 1), -4),
    ]
    for kw, code in cases:
        with pytest.raises(E) as e:
            call(**kw)
        assert _code(e) == code, (kw, str(e.value))


def test_validation_other_entry_points(dm):
    E = dm.DmelError
    with pytest.raises(E) as e:
        dm.dmel_rms_gram(None, 6144, FAKE)
    assert _code(e) == -1
    with pytest.raises(E) as e:
        dm.dmel_rms_gram(FAKE, 6008, FAKE)
    assert _code(e) == -2
    with pytest.raises(E) as e:
        dm.dmel_rms_gram(FAKE, 6144, FAKE, n_bins=81)
    assert _code(e) == -2
    with pytest.raises(E) as e:
        dm.dmel_rms_scale(FAKE, 5, FAKE, 6144, 1e-6, FAKE, n_levels=32)
    assert _code(e) == -2
    with pytest.raises(E) as e:
        dm.dmel_rms_scale(FAKE, 5, FAKE, 6144, -1.0, FAKE)
    assert _code(e) == -1
    with pytest.raises(E) as e:
        dm.dmel_rms_scale(FAKE, 5, FAKE, 6144, float("nan"), FAKE)
    assert _code(e) == -1
    with pytest.raises(E) as e:
        dm.dmel_rms_scale(FAKE + 3, 5, FAKE, 6144, 1e-6, FAKE)
    assert _code(e) == -4
    with pytest.raises(E) as e:
        dm.dmel_gather_rows(FAKE, 10, 12, FAKE, 5, FAKE, 16)
    assert _code(e) == -2
    with pytest.raises(E) as e:
        dm.dmel_gather_rows(FAKE, 10, 16, None, 5, FAKE, 16)
    assert _code(e) == -1
    # forward: workspace too small, gram missing, bad dtype
    args = [None, FAKE, 1600, FAKE, FAKE, 1, 2, None, FAKE, 6144, None, None, 1e-6, FAKE, 0, 6144, None]
    with pytest.raises(E) as e:
        dm.dmel_forward(*args, FAKE, 10)
    assert _code(e) in (-1, -6)
    a = list(args)
    a[0] = None
    with pytest.raises(E) as e:
        dm.dmel_forward(*a, FAKE, dm.dmel_forward_workspace_bytes(2))
    assert _code(e) == -1 and "ctx" in str(e.value)
    with pytest.raises(E) as e:
        dm.dmel_create(-1)
    assert _code(e) in (-1, -5)


def test_validation_training_entry_points(dm):
    """dmel_embed_train and dmel_rms_backward_sums validate before any launch."""
    E = dm.DmelError
    d = 6144
    # embed_train: the dmel_embed checks, then the sums buffer
    with pytest.raises(E) as e:
        dm.dmel_embed_train(FAKE, 5, FAKE, d, None, None, FAKE, dm.DMEL_BF16, d, None, None)
    assert _code(e) == -1 and "sums" in str(e.value)
    with pytest.raises(E) as e:
        dm.dmel_embed_train(FAKE, 5, FAKE, d, None, None, FAKE, dm.DMEL_BF16, d, None, FAKE + 4)
    assert _code(e) == -4
    with pytest.raises(E) as e:
        dm.dmel_embed_train(FAKE, 5, FAKE, 6008, None, None, FAKE, dm.DMEL_BF16, 6008, None, FAKE << 4)
    assert _code(e) == -2
    with pytest.raises(E) as e:  # sums on top of the output
        dm.dmel_embed_train(FAKE, 5, FAKE, d, None, None, FAKE << 8, dm.DMEL_BF16, d, None, (FAKE << 8) + 4096)
    assert _code(e) == -1 and "overlap" in str(e.value)
    dm.dmel_embed_train(None, 0, FAKE, d, None, None, FAKE, dm.DMEL_BF16, d, None, None)  # empty: no-op
    # rms_backward_sums: sizes, dtype, workspace, alignment, overlap
    need = dm.dmel_rms_backward_sums_workspace_bytes(1000, d)
    assert need >= dm.dmel_rms_backward_workspace_bytes(1000, d) + 1000 * 4 and need % 256 == 0
    assert dm.dmel_rms_backward_sums_workspace_bytes(-1, d) == 0
    assert dm.dmel_rms_backward_sums_workspace_bytes(10, 100) == 0
    args = [FAKE << 4, 1000, d, FAKE, FAKE, FAKE << 5, dm.DMEL_BF16, FAKE << 6, None, 0]
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*args, FAKE << 7, need - 1)
    assert _code(e) == -6
    a = list(args); a[2] = 6008
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -2
    a = list(args); a[6] = 7
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -3
    a = list(args); a[0] = None
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -1
    a = list(args); a[3] = None
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -1
    a = list(args); a[0] = (FAKE << 4) + 8
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -4
    a = list(args); a[7] = FAKE << 4  # dsum on top of the sums
    with pytest.raises(E) as e:
        dm.dmel_rms_backward_sums(*a, FAKE << 7, need)
    assert _code(e) == -1 and "overlap" in str(e.value)


def test_validation_shortconv(dm):
    E = dm.DmelError
    C, T, S = 64, 10, 2
    ok = dict(x=FAKE, n_tokens=T, channels=C, seq_off=FAKE, n_seqs=S, weight=FAKE + (1 << 16),
              state_in=None, state_out=None, y=FAKE + (1 << 18), y_dtype=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        dm.dmel_shortconv(a["x"], a["n_tokens"], a["channels"], a["seq_off"], a["n_seqs"], a["weight"],
                          a["state_in"], a["state_out"], a["y"], a["y_dtype"])

    cases = [
        (dict(n_tokens=-1), -1),
        (dict(channels=12), -2),
        (dict(channels=0), -2),
        (dict(n_seqs=0), -2),
        (dict(y_dtype=3), -3),
        (dict(seq_off=None), -1),
        (dict(y=None), -1),
        (dict(weight=None), -1),
        (dict(x=FAKE + 8), -4),
        (dict(seq_off=FAKE + 4), -4),
        (dict(y=FAKE + 96), -1),                      # overlaps x (1280 bytes from FAKE)
        (dict(state_in=FAKE + (1 << 19), state_out=FAKE + (1 << 19)), -1),   # in place
        (dict(state_out=FAKE), -1),                   # overlaps x
    ]
    for kw, code in cases:
        with pytest.raises(E) as e:
            call(**kw)
        assert _code(e) == code, (kw, str(e.value))


def test_zero_work_is_a_noop(dm):
    # T = 0 (short audio) and n_tokens = 0 need no pointers and no GPU
    dm.dmel_embed(None, 0, FAKE, 6144, None, None, FAKE, 0, 6144)
    dm.dmel_rms_scale(None, 0, None, 6144, 1e-6, None)
    dm.dmel_gather_rows(None, 0, 16, None, 0, FAKE, 16)
    dm.dmel_shortconv(None, 0, 64, None, 3, None, None, None, None, 0)


def test_missing_library_fails_loudly(tmp_path):
    code = (
        "import encoder_free_audio_amd.dmel as d\n"
        "d.LIB_PATH = '/nonexistent/libdmel.so'\n"
        "try:\n"
        "    d.dmel_num_frames(16000)\n"
        "except RuntimeError as e:\n"
        "    print('RAISED', e)\n"
    )
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "RAISED" in out.stdout, out.stdout + out.stderr


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "encoder_free_audio_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), fn
                assert "dmel_oracle" not in text, fn


def _bench_header_symbols():
    with open(os.path.join(ROOT, "encoder_free_audio_amd", "csrc", "bench", "dmel_bench.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmel_bench_[a-z_]+)\s*\(", text)))


def test_bench_library_exports(dm):
    # the benchmark-only library loads (after the product library it links
    # against) and exports what its header declares; the product library
    # exports none of it
    from encoder_free_audio_amd import bench_ext as be
    be.lib()
    syms = _bench_header_symbols()
    assert sorted(be.EXPORTS) == syms
    out = subprocess.run(["nm", "-D", "--defined-only", be.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert not [s for s in syms if s not in set(re.findall(r"\bT (dmel_\w+)", out))]
    prod = subprocess.run(["nm", "-D", "--defined-only", dm.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "dft" not in " ".join(re.findall(r"\bT (dmel_\w+)", prod))


def test_dft_gemm_validation(dm):
    # sizes and rejections of the DFT-as-GEMM front end (bench library), in host code
    from encoder_free_audio_amd import bench_ext as be
    assert be.dmel_bench_dft_matrix_bytes() == 1792 * 4800 * 2 + 1792 * 4
    assert be.dmel_bench_dft_gemm_workspace_bytes(0) == 0
    assert be.dmel_bench_dft_gemm_workspace_bytes(1) == 9728 + 7168
    assert be.dmel_bench_dft_gemm_workspace_bytes(1000) == 9_600_000 + 7_168_000
    assert be.dmel_bench_dft_gemm_workspace_bytes(-1) == 0
    E = dm.DmelError
    lib = be.lib()
    with pytest.raises(E) as e:
        be._check("dmel_bench_dft_matrix", lib.dmel_bench_dft_matrix(None, None))
    assert _code(e) == -1
    with pytest.raises(E) as e:
        be._check("dmel_bench_dft_matrix", lib.dmel_bench_dft_matrix(8, None))
    assert _code(e) == -4
    with pytest.raises(E) as e:
        be._check("dmel_bench_rounding_probe", lib.dmel_bench_rounding_probe(256, 512, 1000, 1024, None))
    assert _code(e) == -2
    for fn, top in (("dmel_bench_valu_rate", 16), ("dmel_bench_lds_rate", 3)):
        for bad in ((top + 1, 1, 1, 256), (-1, 1, 1, 256), (0, 0, 1, 256), (0, 1, 0, 256), (0, 1, 1, None)):
            with pytest.raises(E) as e:
                be._check(fn, getattr(lib, fn)(*bad, None))
            assert _code(e) == -1
        with pytest.raises(E) as e:
            be._check(fn, getattr(lib, fn)(0, 1, 1, 2, None))
        assert _code(e) == -4
    # (fake, aligned device addresses: every check fails before any HIP call)
    args = dict(audio=256, n=1600, so=512, fo=768, clips=1, frames=2, carry=None, mat=1024, lm=2048, ws=4096,
                wsb=10 ** 6)

    def call(ctx=None, **kw):
        a = dict(args)
        a.update(kw)
        return lib.dmel_bench_frames_dft_gemm(ctx, a["audio"], a["n"], a["so"], a["fo"], a["clips"], a["frames"],
                                              a["carry"], a["mat"], a["lm"], a["ws"], a["wsb"], None)
    assert call() == -1                                   # NULL context
    assert call(frames=3) == -2                           # more frames than the audio holds
    ctx = dm.dmel_create(0) if dm_has_gpu() else None
    if ctx is not None:
        try:
            assert call(ctx, wsb=100) == -6               # workspace too small
            assert call(ctx, mat=None) == -1
            assert call(ctx, mat=1030) == -4
        finally:
            dm.dmel_destroy(ctx)


def dm_has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
