"""MI355X (gfx950) dMel audio front end: HIP kernels behind the C ABI of
``include/dmel.h`` and a thin ctypes binding (``encoder_free_audio_amd.dmel``)."""

from . import dmel  # noqa: F401
