"""Python face of the C ABI: an encoder handle over torch device tensors.

PyTorch provides device memory and streams only; the forward pass is the
library's kernels, enqueued by aenc_forward on the given stream.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import torch

from . import _lib
from ._lib import AencError, check, lib

TORCH_DTYPE = {_lib.AENC_F32: torch.float32, _lib.AENC_BF16: torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def output_shape(geom) -> Sequence[int]:
    g = _lib.geometry(geom)
    shape = (ctypes.c_int64 * 3)()
    check(lib().aenc_output_shape(ctypes.byref(g), shape), "aenc_output_shape")
    return tuple(int(s) for s in shape)


def param_count(geom) -> int:
    g = _lib.geometry(geom)
    n = lib().aenc_param_count(ctypes.byref(g))
    if n < 0:
        raise AencError(f"aenc_param_count: {_lib.last_error()}")
    return int(n)


def validate(geom) -> int:
    g = _lib.geometry(geom)
    return int(lib().aenc_validate(ctypes.byref(g)))


class Encoder:
    """An encoder on the current HIP device.

    geom: an object with the aenc_geometry fields (batch, n_mel, n_frames,
      d_model, n_layers, n_heads, d_ffn, pool_step, proj_hidden, proj_out,
      dtype, out_dtype, ln_eps, stack, attn_chunk, attn_chunk_mode).
    weights: name -> tensor (host or device, contiguous, the geometry's
      dtype); names conv1_w, conv1_b, conv2_w, conv2_b,
      layers.{l}.{ln1_g, ln1_b, q_w, q_b, k_w, v_w, v_b, o_w, o_b, ln2_g, ln2_b,
      fc1_w, fc1_b, fc2_w, fc2_b}, lnf_g, lnf_b and proj{1,2}_{w,b}. Missing
      biases and betas are zero, missing gammas one.
    The library copies the weights; they may be freed after construction.
    """

    def __init__(self, geom, weights: Dict[str, torch.Tensor]):
        self.geom = geom
        self._g = _lib.geometry(geom)
        check(lib().aenc_validate(ctypes.byref(self._g)), "aenc_validate")
        self.dtype = TORCH_DTYPE[self._g.dtype]
        self.out_dtype = TORCH_DTYPE[self._g.out_dtype]
        keep = []

        def p(name):
            t = weights.get(name)
            if t is None:
                return None
            t = t.contiguous()
            if t.dtype != self.dtype:
                raise ValueError(f"{name}: dtype {t.dtype}, expected {self.dtype}")
            keep.append(t)
            return t.data_ptr()

        layers = (_lib.LayerWeights * max(1, geom.n_layers))()
        for layer in range(geom.n_layers):
            for f in _lib.LAYER_FIELDS:
                setattr(layers[layer], f, p(f"layers.{layer}.{f}"))
        w = _lib.Weights(conv1_w=p("conv1_w"), conv1_b=p("conv1_b"), conv2_w=p("conv2_w"), conv2_b=p("conv2_b"),
                         layers=layers, lnf_g=p("lnf_g"), lnf_b=p("lnf_b"), proj1_w=p("proj1_w"),
                         proj1_b=p("proj1_b"), proj2_w=p("proj2_w"), proj2_b=p("proj2_b"))
        h = lib().aenc_create(ctypes.byref(self._g), ctypes.byref(w))
        if not h:
            raise AencError(f"aenc_create: {_lib.last_error()}")
        self._h = ctypes.c_void_p(h)
        self.out_shape = output_shape(geom)

    def forward(self, mel: torch.Tensor, mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        """Enqueue one forward on `stream` (default: torch's current stream)."""
        g = self._g
        T = g.n_frames // 2
        if tuple(mel.shape) != (g.batch, g.n_mel, g.n_frames) or mel.dtype != self.dtype or not mel.is_cuda:
            raise ValueError(f"mel must be a device tensor {self.dtype} of shape {(g.batch, g.n_mel, g.n_frames)}")
        if mask is not None:
            if tuple(mask.shape) != (g.batch, T) or mask.dtype != torch.uint8 or not mask.is_cuda:
                raise ValueError(f"mask must be a device uint8 tensor of shape {(g.batch, T)}")
        if out is None:
            out = torch.empty(self.out_shape, dtype=self.out_dtype, device=mel.device)
        elif tuple(out.shape) != self.out_shape or out.dtype != self.out_dtype or not out.is_cuda:
            raise ValueError(f"out must be a device tensor {self.out_dtype} of shape {self.out_shape}")
        st = lib().aenc_forward(self._h, _ptr(mel), _ptr(mask), _ptr(out), _stream_handle(stream))
        check(st, "aenc_forward")
        return out

    __call__ = forward

    def forward_cached(self, cache: "EmbeddingsCache", keys, mel: torch.Tensor, mask: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, stream=None):
        """aenc_forward_cached: returns (out, number of clips served from the cache)."""
        g = self._g
        if len(keys) != g.batch:
            raise ValueError(f"need {g.batch} keys")
        if out is None:
            out = torch.empty(self.out_shape, dtype=self.out_dtype, device=mel.device)
        karr = (ctypes.c_uint64 * g.batch)(*[int(k) & 0xFFFFFFFFFFFFFFFF for k in keys])
        hits = ctypes.c_int32(0)
        check(lib().aenc_forward_cached(self._h, cache._c, karr, _ptr(mel), _ptr(mask), _ptr(out),
                                        _stream_handle(stream), ctypes.byref(hits)), "aenc_forward_cached")
        return out, int(hits.value)

    # -- per-step timing -------------------------------------------------
    def profile(self, on: bool = True) -> None:
        check(lib().aenc_profile_enable(self._h, int(on)), "aenc_profile_enable")

    def profile_read(self) -> Dict[str, tuple]:
        """{kind: (total ms, launches)} over the forwards since the last read."""
        n = lib().aenc_profile_kind_count()
        ms = (ctypes.c_double * n)()
        calls = (ctypes.c_int64 * n)()
        got = lib().aenc_profile_read(self._h, ms, calls, n)
        if got < 0:
            check(got, "aenc_profile_read")
        return {lib().aenc_profile_kind_name(k).decode(): (ms[k], calls[k]) for k in range(n) if calls[k]}

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().aenc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class EmbeddingsCache:
    """Device-resident LRU of encoder outputs under 64-bit content keys (aenc_cache_*)."""

    def __init__(self, entry_bytes: int, capacity: int):
        c = lib().aenc_cache_create(int(entry_bytes), int(capacity))
        if not c:
            raise AencError(f"aenc_cache_create: {_lib.last_error()}")
        self._c = ctypes.c_void_p(c)
        self.entry_bytes = int(entry_bytes)

    @classmethod
    def for_encoder(cls, enc: "Encoder", capacity: int) -> "EmbeddingsCache":
        per_clip = enc.out_shape[1] * enc.out_shape[2] * (2 if enc.out_dtype == torch.bfloat16 else 4)
        return cls(per_clip, capacity)

    @staticmethod
    def key_of(data) -> int:
        """A 64-bit content key: BLAKE2b (8-byte digest) of the raw bytes of
        `data` (bytes, a NumPy array or a host tensor), with its shape and dtype
        folded in so that equal bytes of different layouts do not collide."""
        import hashlib
        h = hashlib.blake2b(digest_size=8)
        if isinstance(data, torch.Tensor):
            if data.is_cuda:
                raise ValueError("key_of hashes host data: hash the clip before it is copied to the device")
            t = data.contiguous()
            arr = (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy()
            tag = "bfloat16" if t.dtype == torch.bfloat16 else str(arr.dtype)
            h.update(f"{tag}{tuple(arr.shape)}".encode())
            h.update(arr.tobytes())
        elif hasattr(data, "tobytes"):
            h.update(f"{data.dtype}{tuple(data.shape)}".encode())
            h.update(data.tobytes())
        else:
            h.update(bytes(data))
        return int.from_bytes(h.digest(), "little")

    def __contains__(self, key) -> bool:
        return lib().aenc_cache_contains(self._c, int(key) & 0xFFFFFFFFFFFFFFFF) == 1

    def lookup(self, key, dst: torch.Tensor, stream=None) -> bool:
        st = lib().aenc_cache_lookup(self._c, int(key) & 0xFFFFFFFFFFFFFFFF, _ptr(dst), _stream_handle(stream))
        if st < 0:
            check(st, "aenc_cache_lookup")
        return st == 1

    def insert(self, key, src: torch.Tensor, stream=None) -> None:
        check(lib().aenc_cache_insert(self._c, int(key) & 0xFFFFFFFFFFFFFFFF, _ptr(src), _stream_handle(stream)),
              "aenc_cache_insert")

    def stats(self) -> Dict[str, int]:
        out = (ctypes.c_int64 * 5)()
        check(lib().aenc_cache_stats(self._c, out), "aenc_cache_stats")
        return dict(zip(("hits", "misses", "inserts", "evictions", "entries"), (int(v) for v in out)))

    def close(self):
        if getattr(self, "_c", None):
            lib().aenc_cache_destroy(self._c)
            self._c = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
