"""Python face of the log-mel front end (aenc_frontend_* in include/aenc.h).

Audio in, encoder features out, on the GPU: the binding only marshals
arguments; the work is the library's kernels on the given stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import AencError, check, lib
from .encoder import _ptr, _stream_handle

TORCH_DTYPE = {_lib.AENC_F32: torch.float32, _lib.AENC_BF16: torch.bfloat16}


def _config(batch: int, n_samples: int, n_mel: int, out_dtype) -> _lib.FrontendConfig:
    return _lib.FrontendConfig(batch=batch, n_samples=n_samples, n_mel=n_mel, out_dtype=_lib.dtype_code(out_dtype))


def frontend_output_shape(batch: int, n_samples: int = 480000, n_mel: int = 128, out_dtype="bf16") -> Tuple[int, ...]:
    c = _config(batch, n_samples, n_mel, out_dtype)
    shape = (ctypes.c_int64 * 3)()
    check(lib().aenc_frontend_output_shape(ctypes.byref(c), shape), "aenc_frontend_output_shape")
    return tuple(int(s) for s in shape)


class Frontend:
    """16 kHz audio [batch, n_samples] fp32 -> features [batch, n_mel, n_samples / 160]."""

    def __init__(self, batch: int, n_samples: int = 480000, n_mel: int = 128, out_dtype="bf16"):
        self.cfg = _config(batch, n_samples, n_mel, out_dtype)
        self.out_shape = frontend_output_shape(batch, n_samples, n_mel, out_dtype)
        self.out_dtype = TORCH_DTYPE[self.cfg.out_dtype]
        h = lib().aenc_frontend_create(ctypes.byref(self.cfg))
        if not h:
            raise AencError(f"aenc_frontend_create: {_lib.last_error()}")
        self._h = ctypes.c_void_p(h)

    def __call__(self, audio: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if audio.dtype != torch.float32 or tuple(audio.shape) != (self.cfg.batch, self.cfg.n_samples):
            raise ValueError(f"audio must be float32 [{self.cfg.batch}, {self.cfg.n_samples}]")
        if out is None:
            out = torch.empty(self.out_shape, dtype=self.out_dtype, device=audio.device)
        elif out.dtype != self.out_dtype or tuple(out.shape) != self.out_shape:
            raise ValueError(f"out must be {self.out_dtype} {self.out_shape}")
        check(lib().aenc_frontend_run(self._h, _ptr(audio), _ptr(out), _stream_handle(stream)), "aenc_frontend_run")
        return out

    def close(self):
        if getattr(self, "_h", None):
            lib().aenc_frontend_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
