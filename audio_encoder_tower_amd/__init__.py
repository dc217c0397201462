"""MI355X-native Whisper-style audio encoder tower.

The forward pass runs in hand-written HIP kernels for gfx950 behind the C ABI
of include/aenc.h (libaenc.so); this package is its Python binding.
"""
from ._lib import AencError, AENC_BF16, AENC_F32, lib, last_error  # noqa: F401
from .encoder import EmbeddingsCache, Encoder, output_shape, param_count, validate  # noqa: F401
from .frontend import Frontend, frontend_output_shape  # noqa: F401
from . import steps  # noqa: F401
