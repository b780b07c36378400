"""ctypes binding of libdmel (include/dmel.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors (device memory) or plain ints, passes their data pointers and the
current HIP stream, and raises :class:`DmelError` when the call returns an
error.  No step of the front end runs in Python: if the library is missing
the import of a binding function fails loudly.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libdmel.so")

DMEL_BF16 = 0
DMEL_F32 = 1

_STATUS = {0: "DMEL_OK", -1: "DMEL_EINVAL", -2: "DMEL_ESHAPE", -3: "DMEL_EDTYPE", -4: "DMEL_EALIGN",
           -5: "DMEL_EHIP", -6: "DMEL_ENOMEM", -7: "DMEL_ESTATE"}

# Every symbol include/dmel.h declares.
EXPORTS = ("dmel_get_params", "dmel_num_frames", "dmel_last_error", "dmel_default_config", "dmel_create",
           "dmel_create_config", "dmel_get_config", "dmel_destroy", "dmel_frames", "dmel_levels", "dmel_rms_gram",
           "dmel_rms_scale", "dmel_embed", "dmel_embed_train", "dmel_forward_workspace_bytes", "dmel_forward",
           "dmel_forward_noalloc",
           "dmel_gather_rows",
           "dmel_shortconv", "dmel_embed_backward_workspace_bytes", "dmel_embed_backward",
           "dmel_rms_backward_workspace_bytes", "dmel_rms_backward_stored_workspace_bytes", "dmel_rms_backward",
           "dmel_rms_backward_sums_workspace_bytes", "dmel_rms_backward_sums",
           "dmel_hmlp_workspace_bytes",
           "dmel_hmlp_forward", "dmel_hmlp_stage")


class DmelError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {_STATUS.get(code, code)}: {msg}")
        self.code = code
        self.fn = fn


class DmelParams(ctypes.Structure):
    _fields_ = [("sample_rate", ctypes.c_int32), ("hop", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_fft", ctypes.c_int32), ("n_bins", ctypes.c_int32), ("n_mels", ctypes.c_int32),
                ("n_levels", ctypes.c_int32), ("n_rows", ctypes.c_int32), ("clamp_min", ctypes.c_float),
                ("clamp_max", ctypes.c_float), ("log_floor", ctypes.c_float), ("f_min_hz", ctypes.c_float),
                ("f_max_hz", ctypes.c_float)]


class DmelConfig(ctypes.Structure):
    _fields_ = [("n_mel_bins", ctypes.c_int32), ("mel_vocab_size", ctypes.c_int32), ("min_value", ctypes.c_float),
                ("max_value", ctypes.c_float)]


_lib_handle = None
_lib_lock = threading.Lock()

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libdmel.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    with _lib_lock:
        if _lib_handle is not None:
            return _lib_handle
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m encoder_free_audio_amd.build)")
        h = ctypes.CDLL(LIB_PATH)
        sig = {
            "dmel_get_params": (ctypes.c_int, [ctypes.POINTER(DmelParams)]),
            "dmel_num_frames": (_I64, [_I64]),
            "dmel_last_error": (ctypes.c_char_p, []),
            "dmel_default_config": (ctypes.c_int, [ctypes.POINTER(DmelConfig)]),
            "dmel_create": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int]),
            "dmel_create_config": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int, ctypes.POINTER(DmelConfig)]),
            "dmel_get_config": (ctypes.c_int, [_P, ctypes.POINTER(DmelConfig)]),
            "dmel_destroy": (ctypes.c_int, [_P]),
            "dmel_frames": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P]),
            "dmel_levels": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P]),
            "dmel_rms_gram": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P]),
            "dmel_rms_scale": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _F, _P, _P]),
            "dmel_embed": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _I64, _P, _P]),
            "dmel_embed_train": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _I64, _P, _P, _P]),
            "dmel_forward_workspace_bytes": (_SZ, [_I64]),
            "dmel_forward": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _I32, _P, _P, _F,
                                            _P, _I32, _I64, _P, _P, _SZ, _P]),
            "dmel_forward_noalloc": (ctypes.c_int, [_P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _I32, _P, _P, _F,
                                                    _P, _I32, _I64, _P, _P]),
            "dmel_gather_rows": (ctypes.c_int, [_P, _I64, _I32, _P, _I64, _P, _I64, _P, _P]),
            "dmel_shortconv": (ctypes.c_int, [_P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _I32, _P]),
            "dmel_embed_backward_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32]),
            "dmel_embed_backward": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _I32, _P, _I32, _P, _SZ, _P]),
            "dmel_rms_backward_workspace_bytes": (_SZ, [_I64, _I32]),
            "dmel_rms_backward_stored_workspace_bytes": (_SZ, [_I64, _I32]),
            "dmel_hmlp_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
            "dmel_hmlp_forward": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P,
                                                 _I32, _P, _SZ, _P]),
            "dmel_hmlp_stage": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, _I32, _P, _I32, _P]),
            "dmel_rms_backward": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _P, _P, _I32, _P,
                                                 _SZ, _P]),
            "dmel_rms_backward_sums_workspace_bytes": (_SZ, [_I64, _I32]),
            "dmel_rms_backward_sums": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _I32, _P, _P, _I32, _P, _SZ, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
        return h


def _check(fn: str, rc: int):
    if rc != 0:
        raise DmelError(fn, rc, lib().dmel_last_error().decode(errors="replace"))


def _ptr(t) -> int | None:
    """Data pointer of a tensor (None -> NULL).  Raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def dmel_get_params() -> dict:
    p = DmelParams()
    _check("dmel_get_params", lib().dmel_get_params(ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in DmelParams._fields_}


def dmel_num_frames(n_samples: int) -> int:
    return int(lib().dmel_num_frames(int(n_samples)))


def dmel_last_error() -> str:
    return lib().dmel_last_error().decode(errors="replace")


def dmel_default_config() -> dict:
    c = DmelConfig()
    _check("dmel_default_config", lib().dmel_default_config(ctypes.byref(c)))
    return {name: getattr(c, name) for name, _ in DmelConfig._fields_}


def dmel_create(device: int = 0) -> int:
    """Returns the context handle (an int) for HIP device ``device``."""
    h = _P()
    _check("dmel_create", lib().dmel_create(ctypes.byref(h), int(device)))
    return h.value


def dmel_create_config(device: int = 0, config: dict | None = None) -> int:
    """Context with the configuration ``config`` (keys of DmelConfig; None: released)."""
    h = _P()
    c = None
    if config is not None:
        c = DmelConfig(int(config["n_mel_bins"]), int(config["mel_vocab_size"]), float(config["min_value"]),
                       float(config["max_value"]))
    _check("dmel_create_config",
           lib().dmel_create_config(ctypes.byref(h), int(device), ctypes.byref(c) if c is not None else None))
    return h.value


def dmel_get_config(ctx) -> dict:
    c = DmelConfig()
    _check("dmel_get_config", lib().dmel_get_config(ctx, ctypes.byref(c)))
    return {name: getattr(c, name) for name, _ in DmelConfig._fields_}


def dmel_destroy(ctx: int) -> None:
    _check("dmel_destroy", lib().dmel_destroy(ctx))


def dmel_frames(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, logmel,
                stream=None) -> None:
    _check("dmel_frames", lib().dmel_frames(ctx, _ptr(audio), int(n_samples_total), _ptr(sample_off),
                                            _ptr(frame_off), int(n_clips), int(n_frames_total), _ptr(carry),
                                            _ptr(logmel), _stream(stream)))


def dmel_levels(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, levels,
                stream=None) -> None:
    _check("dmel_levels", lib().dmel_levels(ctx, _ptr(audio), int(n_samples_total), _ptr(sample_off),
                                            _ptr(frame_off), int(n_clips), int(n_frames_total), _ptr(carry),
                                            _ptr(levels), _stream(stream)))


# The table layout (n_bins, n_levels) of the next three calls is keyword-only
# here and defaults to the released 80 x 16; the C arguments keep their order.
def dmel_rms_gram(table, d_model, gram, stream=None, *, n_bins=80, n_levels=16) -> None:
    _check("dmel_rms_gram", lib().dmel_rms_gram(_ptr(table), int(n_bins), int(n_levels), int(d_model), _ptr(gram),
                                                _stream(stream)))


def dmel_rms_scale(levels, n_tokens, gram, d_model, eps, scale, stream=None, *, n_bins=80, n_levels=16) -> None:
    _check("dmel_rms_scale", lib().dmel_rms_scale(_ptr(levels), int(n_tokens), int(n_bins), int(n_levels),
                                                  _ptr(gram), int(d_model), float(eps), _ptr(scale),
                                                  _stream(stream)))


def dmel_embed(levels, n_tokens, table, d_model, rms_weight, rms_scale, out, out_dtype, out_row_stride,
               out_rows=None, stream=None, *, n_bins=80, n_levels=16) -> None:
    _check("dmel_embed", lib().dmel_embed(_ptr(levels), int(n_tokens), int(n_bins), int(n_levels), _ptr(table),
                                          int(d_model), _ptr(rms_weight), _ptr(rms_scale), _ptr(out),
                                          int(out_dtype), int(out_row_stride), _ptr(out_rows), _stream(stream)))


def dmel_embed_train(levels, n_tokens, table, d_model, rms_weight, rms_scale, out, out_dtype, out_row_stride,
                     out_rows, sums, stream=None, *, n_bins=80, n_levels=16) -> None:
    _check("dmel_embed_train", lib().dmel_embed_train(_ptr(levels), int(n_tokens), int(n_bins), int(n_levels),
                                                      _ptr(table), int(d_model), _ptr(rms_weight), _ptr(rms_scale),
                                                      _ptr(out), int(out_dtype), int(out_row_stride),
                                                      _ptr(out_rows), _ptr(sums), _stream(stream)))


def dmel_forward_workspace_bytes(n_frames_total: int) -> int:
    return int(lib().dmel_forward_workspace_bytes(int(n_frames_total)))


def dmel_forward(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                 d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows, workspace,
                 workspace_bytes, stream=None) -> None:
    _check("dmel_forward", lib().dmel_forward(ctx, _ptr(audio), int(n_samples_total), _ptr(sample_off),
                                              _ptr(frame_off), int(n_clips), int(n_frames_total), _ptr(carry),
                                              _ptr(table), int(d_model), _ptr(rms_weight), _ptr(gram),
                                              float(eps), _ptr(out), int(out_dtype), int(out_row_stride),
                                              _ptr(out_rows), _ptr(workspace), int(workspace_bytes),
                                              _stream(stream)))


# Largest batch dmel_forward_noalloc accepts (DMEL_NOALLOC_MAX_FRAMES).
NOALLOC_MAX_FRAMES = 262144


def dmel_forward_noalloc(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                         d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows,
                         stream=None) -> None:
    _check("dmel_forward_noalloc",
           lib().dmel_forward_noalloc(ctx, _ptr(audio), int(n_samples_total), _ptr(sample_off), _ptr(frame_off),
                                      int(n_clips), int(n_frames_total), _ptr(carry), _ptr(table), int(d_model),
                                      _ptr(rms_weight), _ptr(gram), float(eps), _ptr(out), int(out_dtype),
                                      int(out_row_stride), _ptr(out_rows), _stream(stream)))


def dmel_gather_rows(table, n_table_rows, d_model, ids, n, out, out_row_stride, out_rows=None,
                     stream=None) -> None:
    _check("dmel_gather_rows", lib().dmel_gather_rows(_ptr(table), int(n_table_rows), int(d_model), _ptr(ids),
                                                      int(n), _ptr(out), int(out_row_stride), _ptr(out_rows),
                                                      _stream(stream)))


def dmel_shortconv(x, n_tokens, channels, seq_off, n_seqs, weight, state_in, state_out, y, y_dtype,
                   stream=None) -> None:
    _check("dmel_shortconv", lib().dmel_shortconv(_ptr(x), int(n_tokens), int(channels), _ptr(seq_off), int(n_seqs),
                                                  _ptr(weight), _ptr(state_in), _ptr(state_out), _ptr(y),
                                                  int(y_dtype), _stream(stream)))


def dmel_embed_backward_workspace_bytes(n_tokens, n_bins, n_levels, d_model) -> int:
    return int(lib().dmel_embed_backward_workspace_bytes(int(n_tokens), int(n_bins), int(n_levels), int(d_model)))


def dmel_embed_backward(levels, n_tokens, n_bins, n_levels, dsum, dsum_dtype, d_model, dtable, accumulate, workspace,
                        workspace_bytes, stream=None) -> None:
    _check("dmel_embed_backward", lib().dmel_embed_backward(_ptr(levels), int(n_tokens), int(n_bins), int(n_levels),
                                                            _ptr(dsum), int(dsum_dtype), int(d_model), _ptr(dtable),
                                                            int(accumulate), _ptr(workspace), int(workspace_bytes),
                                                            _stream(stream)))


def dmel_rms_backward_workspace_bytes(n_tokens, d_model) -> int:
    return int(lib().dmel_rms_backward_workspace_bytes(int(n_tokens), int(d_model)))


def dmel_rms_backward_stored_workspace_bytes(n_tokens, d_model) -> int:
    return int(lib().dmel_rms_backward_stored_workspace_bytes(int(n_tokens), int(d_model)))


def dmel_rms_backward(levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, dy, dy_dtype, dsum,
                      dweight, accumulate_dweight, workspace, workspace_bytes, stream=None) -> None:
    _check("dmel_rms_backward", lib().dmel_rms_backward(_ptr(levels), int(n_tokens), int(n_bins), int(n_levels),
                                                        _ptr(table), int(d_model), _ptr(rms_weight), _ptr(rms_scale),
                                                        _ptr(dy), int(dy_dtype), _ptr(dsum), _ptr(dweight),
                                                        int(accumulate_dweight), _ptr(workspace),
                                                        int(workspace_bytes), _stream(stream)))


def dmel_rms_backward_sums_workspace_bytes(n_tokens, d_model) -> int:
    return int(lib().dmel_rms_backward_sums_workspace_bytes(int(n_tokens), int(d_model)))


def dmel_rms_backward_sums(sums, n_tokens, d_model, rms_weight, rms_scale, dy, dy_dtype, dsum, dweight,
                           accumulate_dweight, workspace, workspace_bytes, stream=None) -> None:
    _check("dmel_rms_backward_sums",
           lib().dmel_rms_backward_sums(_ptr(sums), int(n_tokens), int(d_model), _ptr(rms_weight), _ptr(rms_scale),
                                        _ptr(dy), int(dy_dtype), _ptr(dsum), _ptr(dweight), int(accumulate_dweight),
                                        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def dmel_hmlp_workspace_bytes(n_images, height, width, hidden) -> int:
    return int(lib().dmel_hmlp_workspace_bytes(int(n_images), int(height), int(width), int(hidden)))


def dmel_hmlp_forward(images, n_images, height, width, w1, b1, w2, b2, w3, b3, w4, b4, hidden, d_model, out, out_dtype,
                      workspace, workspace_bytes, stream=None) -> None:
    _check("dmel_hmlp_forward", lib().dmel_hmlp_forward(_ptr(images), int(n_images), int(height), int(width), _ptr(w1),
                                                        _ptr(b1), _ptr(w2), _ptr(b2), _ptr(w3), _ptr(b3), _ptr(w4),
                                                        _ptr(b4), int(hidden), int(d_model), _ptr(out), int(out_dtype),
                                                        _ptr(workspace), int(workspace_bytes), _stream(stream)))


def dmel_hmlp_stage(x, n_rows, k, weight, bias, n, gelu, y, y_dtype, stream=None) -> None:
    _check("dmel_hmlp_stage", lib().dmel_hmlp_stage(_ptr(x), int(n_rows), int(k), _ptr(weight), _ptr(bias), int(n),
                                                    int(gelu), _ptr(y), int(y_dtype), _stream(stream)))


# ---------------------------------------------------------------------------
# Marshalling helpers: offsets for ragged clips, allocation of outputs.
# ---------------------------------------------------------------------------
def clip_offsets(lengths, device) -> tuple[torch.Tensor, torch.Tensor, int]:
    """(sample_off, frame_off, n_frames_total) device int64 tensors for clip lengths."""
    lengths = [int(v) for v in lengths]
    s_off = [0]
    f_off = [0]
    for n in lengths:
        s_off.append(s_off[-1] + n)
        f_off.append(f_off[-1] + dmel_num_frames(n))
    so = torch.tensor(s_off, dtype=torch.int64, device=device)
    fo = torch.tensor(f_off, dtype=torch.int64, device=device)
    return so, fo, f_off[-1]
