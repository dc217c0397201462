"""ctypes view of libaenc.so (include/aenc.h and include/aenc_kernels.h).

Argument marshalling only: every step of the encoder runs in the library's
HIP kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
# AENC_LIBRARY may name another build of the same library (the host-sanitizer
# copy that `python -m audio_encoder_tower_amd.build --sanitize` writes).
LIB_PATH = os.environ.get("AENC_LIBRARY") or os.path.join(PKG, "libaenc.so")

AENC_F32 = 0
AENC_BF16 = 1
# bytes of the static scratch array of aenc_forward_noalloc (AENC_NOALLOC_SCRATCH_BYTES)
AENC_NOALLOC_SCRATCH_BYTES = 96 << 20

STATUS = {0: "AENC_OK", -1: "AENC_E_INVAL", -2: "AENC_E_UNSUPPORTED", -3: "AENC_E_NOMEM",
          -4: "AENC_E_DEVICE", -5: "AENC_E_HIP"}


class Geometry(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_mel", c_int32), ("n_frames", c_int32), ("d_model", c_int32),
                ("n_layers", c_int32), ("n_heads", c_int32), ("d_ffn", c_int32), ("pool_step", c_int32),
                ("proj_hidden", c_int32), ("proj_out", c_int32), ("dtype", c_int32), ("out_dtype", c_int32),
                ("ln_eps", c_float), ("stack", c_int32), ("attn_chunk", c_int32), ("attn_chunk_mode", c_int32)]


LAYER_FIELDS = ("ln1_g", "ln1_b", "q_w", "q_b", "k_w", "v_w", "v_b", "o_w", "o_b",
                "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("conv1_w", c_void_p), ("conv1_b", c_void_p), ("conv2_w", c_void_p), ("conv2_b", c_void_p),
                ("layers", POINTER(LayerWeights)), ("lnf_g", c_void_p), ("lnf_b", c_void_p),
                ("proj1_w", c_void_p), ("proj1_b", c_void_p), ("proj2_w", c_void_p), ("proj2_b", c_void_p)]


class FrontendConfig(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_samples", c_int32), ("n_mel", c_int32), ("out_dtype", c_int32)]


class AencError(RuntimeError):
    pass


_lib = None

SIGNATURES = {
    # aenc.h
    "aenc_validate": (c_int, [POINTER(Geometry)]),
    "aenc_create": (c_void_p, [POINTER(Geometry), POINTER(Weights)]),
    "aenc_forward": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "aenc_destroy": (None, [c_void_p]),
    "aenc_last_error": (c_char_p, []),
    "aenc_param_count": (c_int64, [POINTER(Geometry)]),
    "aenc_output_shape": (c_int, [POINTER(Geometry), POINTER(c_int64)]),
    "aenc_workspace_bytes": (c_int64, [POINTER(Geometry)]),
    "aenc_profile_enable": (c_int, [c_void_p, c_int]),
    "aenc_profile_read": (c_int, [c_void_p, POINTER(c_double), POINTER(c_int64), c_int]),
    "aenc_profile_kind_count": (c_int, []),
    "aenc_profile_kind_name": (c_char_p, [c_int]),
    # aenc_kernels.h
    "aenc_k_gemm_bf16": (c_int, [c_int, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int,
                                 c_int, c_int, c_void_p]),
    "aenc_k_qkv_bf16": (c_int, [c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_int64, c_int, c_int,
                                c_void_p]),
    "aenc_k_attention_bf16": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p, c_void_p]),
    "aenc_k_chunk_ranges": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p]),
    "aenc_k_layernorm": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_float, c_void_p]),
    "aenc_k_gelu_f32": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "aenc_k_row_maps": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]),
    "aenc_k_copy": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "aenc_k_copy_stream": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "aenc_k_mfma_loop": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "aenc_k_row_stream": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "aenc_handle_geometry": (c_int, [c_void_p, POINTER(Geometry)]),
    "aenc_forward_noalloc": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "aenc_noalloc_scratch_bytes": (c_int64, [POINTER(Geometry), c_int]),
    # embeddings cache (aenc.h)
    "aenc_cache_create": (c_void_p, [c_int64, c_int64]),
    "aenc_cache_destroy": (None, [c_void_p]),
    "aenc_cache_contains": (c_int, [c_void_p, ctypes.c_uint64]),
    "aenc_cache_lookup": (c_int, [c_void_p, ctypes.c_uint64, c_void_p, c_void_p]),
    "aenc_cache_insert": (c_int, [c_void_p, ctypes.c_uint64, c_void_p, c_void_p]),
    "aenc_cache_stats": (c_int, [c_void_p, POINTER(c_int64)]),
    "aenc_forward_cached": (c_int, [c_void_p, c_void_p, POINTER(ctypes.c_uint64), c_void_p, c_void_p, c_void_p,
                                    c_void_p, POINTER(ctypes.c_int32)]),
    # front end (aenc.h)
    "aenc_frontend_output_shape": (c_int, [POINTER(FrontendConfig), POINTER(c_int64)]),
    "aenc_frontend_create": (c_void_p, [POINTER(FrontendConfig)]),
    "aenc_frontend_run": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p]),
    "aenc_frontend_destroy": (None, [c_void_p]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libaenc.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise AencError(f"{LIB_PATH} is missing: build it with `python -m audio_encoder_tower_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    msg = lib().aenc_last_error()
    return msg.decode() if msg else ""


def check(status: int, what: str) -> None:
    if status != 0:
        raise AencError(f"{what}: {STATUS.get(status, status)}: {last_error()}")


def dtype_code(x) -> int:
    if x in (AENC_F32, AENC_BF16):
        return int(x)
    s = str(x).lower()
    if "bf16" in s or "bfloat16" in s:
        return AENC_BF16
    if "f32" in s or "float32" in s:
        return AENC_F32
    raise ValueError(f"unsupported dtype {x!r}")


def geometry(g) -> Geometry:
    """Build the C geometry from any object with the aenc_geometry field names."""
    return Geometry(batch=g.batch, n_mel=g.n_mel, n_frames=g.n_frames, d_model=g.d_model,
                    n_layers=g.n_layers, n_heads=g.n_heads, d_ffn=g.d_ffn, pool_step=g.pool_step,
                    proj_hidden=g.proj_hidden, proj_out=g.proj_out, dtype=dtype_code(g.dtype),
                    out_dtype=dtype_code(g.out_dtype), ln_eps=g.ln_eps,
                    stack=getattr(g, "stack", 1), attn_chunk=getattr(g, "attn_chunk", 0),
                    attn_chunk_mode=getattr(g, "attn_chunk_mode", 0))
