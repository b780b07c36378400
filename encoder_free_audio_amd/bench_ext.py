"""ctypes binding of libdmel_bench (csrc/bench/dmel_bench.h), the
benchmark-only companion of libdmel: the DFT-as-matrix-product log-mel that
the FFT front end was measured against, the rounding probe and the
vector-ALU issue-rate calibration.  Argument
marshalling only; only bench.py and the tests load it."""

from __future__ import annotations

import ctypes
import os
import threading

from encoder_free_audio_amd import dmel as _dm

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdmel_bench.so")
EXPORTS = ("dmel_bench_last_error", "dmel_bench_dft_matrix_bytes", "dmel_bench_dft_matrix",
           "dmel_bench_dft_gemm_workspace_bytes", "dmel_bench_frames_dft_gemm", "dmel_bench_rounding_probe",
           "dmel_bench_valu_rate", "dmel_bench_lds_rate")

_handle = None
_lock = threading.Lock()
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _handle
    if _handle is not None:
        return _handle
    with _lock:
        if _handle is None:
            _dm.lib()   # the product library first (the bench library links against it)
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m encoder_free_audio_amd.build)")
            h = ctypes.CDLL(LIB_PATH)
            sig = {
                "dmel_bench_last_error": (ctypes.c_char_p, []),
                "dmel_bench_dft_matrix_bytes": (_SZ, []),
                "dmel_bench_dft_matrix": (ctypes.c_int, [_P, _P]),
                "dmel_bench_dft_gemm_workspace_bytes": (_SZ, [_I64]),
                "dmel_bench_frames_dft_gemm": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P, _P,
                                                              _SZ, _P]),
                "dmel_bench_rounding_probe": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
                "dmel_bench_valu_rate": (ctypes.c_int, [_I32, _I32, _I32, _P, _P]),
                "dmel_bench_lds_rate": (ctypes.c_int, [_I32, _I32, _I32, _P, _P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _handle = h
    return _handle


def _check(fn: str, rc: int):
    if rc != 0:
        raise _dm.DmelError(fn, rc, lib().dmel_bench_last_error().decode(errors="replace"))


def dmel_bench_dft_matrix_bytes() -> int:
    return int(lib().dmel_bench_dft_matrix_bytes())


def dmel_bench_dft_matrix(matrix, stream=None) -> None:
    _check("dmel_bench_dft_matrix", lib().dmel_bench_dft_matrix(_dm._ptr(matrix), _dm._stream(stream)))


def dmel_bench_dft_gemm_workspace_bytes(n_frames_total: int) -> int:
    return int(lib().dmel_bench_dft_gemm_workspace_bytes(int(n_frames_total)))


def dmel_bench_frames_dft_gemm(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry,
                               matrix, logmel, workspace, workspace_bytes, stream=None) -> None:
    p = _dm._ptr
    _check("dmel_bench_frames_dft_gemm",
           lib().dmel_bench_frames_dft_gemm(ctx, p(audio), int(n_samples_total), p(sample_off), p(frame_off),
                                            int(n_clips), int(n_frames_total), p(carry), p(matrix), p(logmel),
                                            p(workspace), int(workspace_bytes), _dm._stream(stream)))


def dmel_bench_rounding_probe(c, e, n, out, stream=None) -> None:
    p = _dm._ptr
    _check("dmel_bench_rounding_probe", lib().dmel_bench_rounding_probe(p(c), p(e), int(n), p(out),
                                                                        _dm._stream(stream)))


def dmel_bench_valu_rate(kind, blocks, iters, out, stream=None) -> None:
    _check("dmel_bench_valu_rate", lib().dmel_bench_valu_rate(int(kind), int(blocks), int(iters), _dm._ptr(out),
                                                              _dm._stream(stream)))


def dmel_bench_lds_rate(mode, blocks, iters, out, stream=None) -> None:
    _check("dmel_bench_lds_rate", lib().dmel_bench_lds_rate(int(mode), int(blocks), int(iters), _dm._ptr(out),
                                                            _dm._stream(stream)))
