"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every declared symbol, geometry validation and the closed forms."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("aenc.h", "aenc_kernels.h")]


@pytest.fixture(scope="module")
def aenc():
    import audio_encoder_tower_amd as a
    a.lib()
    return a


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(aenc_\w+)\s*\(", text)
    return sorted(set(names))


def test_headers_compile_as_c_and_cxx():
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        for h in HEADERS:
            subprocess.run(["gcc", "-fsyntax-only", "-Wall", "-Werror", "-x", lang, std, h], check=True)


def test_library_exports_every_declared_symbol(aenc):
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(aenc.lib(), n)]
    assert not missing, missing
    # and the binding gives each a signature
    from audio_encoder_tower_amd._lib import SIGNATURES
    assert set(names) == set(SIGNATURES)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workloads_validate_and_match_closed_forms(aenc, name):
    g = synth.get_workload(name).geom
    assert aenc.validate(g) == 0
    assert aenc.param_count(g) == oracle.param_count(g)
    assert aenc.output_shape(g) == (g.batch, g.t_out, g.d_out)
    gg = aenc._lib.geometry(g)
    assert aenc.lib().aenc_workspace_bytes(ctypes.byref(gg)) > 0


BAD = {
    "batch0": dict(batch=0),
    "odd_frames": dict(n_frames=301),
    "too_many_frames": dict(n_frames=3002),
    "head_dim_not_64": dict(n_heads=5),
    "d_not_mult_128": dict(d_model=192, n_heads=3),
    "ffn_not_mult_64": dict(d_ffn=1000),
    "pool3": dict(pool_step=3),
    "proj_half": dict(proj_hidden=64, proj_out=0),
    "bad_dtype": dict(dtype="f16"),
    "eps0": dict(ln_eps=0.0),
    "eps_nan": dict(ln_eps=float("nan")),
    "neg_layers": dict(n_layers=-1),
    "stack3": dict(stack=3, proj_hidden=128, proj_out=128),
    "stack4_too_short": dict(stack=4, proj_hidden=128, proj_out=128, n_frames=6),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_invalid_geometries_are_rejected(aenc, case):
    g = synth.get_workload("whisper_large_b1").geom
    kw = dict(BAD[case])
    if kw.get("dtype") == "f16":
        gg = aenc._lib.geometry(g)
        gg.dtype = 7
        assert aenc.lib().aenc_validate(ctypes.byref(gg)) == -1
        return
    assert aenc.validate(g.replace(**kw)) == -1, case
    assert aenc.last_error()
    assert aenc.lib().aenc_param_count(ctypes.byref(aenc._lib.geometry(g.replace(**kw)))) == -1


def test_bf16_batch_limit_of_32_bit_gemm_offsets(aenc):
    """The bf16 GEMMs reach their operands through 32-bit byte offsets. For
    Whisper-large the FFN hidden rows are the largest operand: 1504 padded rows
    x 5120 x 2 bytes = 15,400,960 bytes per clip, so 278 clips fit under
    4 GiB and 279 do not; validation names the limit."""
    g = synth.get_workload("whisper_large_b1").geom
    assert aenc.validate(g.replace(batch=278)) == 0
    assert aenc.validate(g.replace(batch=279)) == -1
    assert "at most 278 clips" in aenc.last_error()
    # a projector hidden width above d_ffn sets the limit instead
    gp = g.replace(proj_hidden=8192, proj_out=64)
    per_clip = 1504 * 8192 * 2
    ok = (2**32 - 2) // per_clip
    assert aenc.validate(gp.replace(batch=ok)) == 0
    assert aenc.validate(gp.replace(batch=ok + 1)) == -1


def test_pool_with_projector_is_unsupported(aenc):
    g = synth.get_workload("whisper_medium_pool2_b1").geom.replace(proj_hidden=128, proj_out=128)
    assert aenc.validate(g) == -2
    assert "pool" in aenc.last_error()


def test_stacking_needs_a_projector(aenc):
    g = synth.get_workload("whisper_large_b1").geom.replace(stack=4)
    assert aenc.validate(g) == -2
    assert "projector" in aenc.last_error()
    g = synth.get_workload("whisper_medium_pool2_b1").geom.replace(stack=4, proj_hidden=128, proj_out=128)
    assert aenc.validate(g) == -2


def test_stacked_geometry_counts(aenc):
    """stack 4: 375 output rows per 30 s clip and a 4 d-wide projector input,
    the same closed forms on both sides of the boundary."""
    g = synth.get_workload("whisper_large_stack4_proj_b16").geom
    assert aenc.output_shape(g) == (16, 375, 3072)
    assert aenc.param_count(g) - aenc.param_count(g.replace(stack=1)) == 3 * 1280 * 3072
    # a zero stack field (a caller that predates it) means no stacking
    gg = aenc._lib.geometry(g.replace(stack=1))
    gg.stack = 0
    assert aenc.lib().aenc_validate(ctypes.byref(gg)) == 0


def test_frontend_shapes_and_configs(aenc):
    assert aenc.frontend_output_shape(16, 480000, 128) == (16, 128, 3000)     # 30 s -> 3000 frames
    assert aenc.frontend_output_shape(2, 80000, 80, "f32") == (2, 80, 500)
    for bad in (dict(batch=0), dict(n_samples=1000), dict(n_samples=160), dict(n_mel=0), dict(n_mel=600)):
        kw = dict(batch=1, n_samples=16000, n_mel=128)
        kw.update(bad)
        with pytest.raises(aenc.AencError):
            aenc.frontend_output_shape(**kw)
    L = aenc.lib()
    assert L.aenc_frontend_create(None) is None
    assert L.aenc_frontend_run(None, None, None, None) == -1
    L.aenc_frontend_destroy(None)


def test_null_arguments(aenc):
    L = aenc.lib()
    assert L.aenc_validate(None) == -1
    assert L.aenc_create(None, None) is None
    assert L.aenc_forward(None, None, None, None, None) == -1
    L.aenc_destroy(None)
    g = aenc._lib.geometry(synth.get_workload("tiny_fp32_b1").geom)
    assert L.aenc_create(ctypes.byref(g), None) is None
    assert "weights" in aenc.last_error()
    assert L.aenc_output_shape(ctypes.byref(g), None) == -1
    assert L.aenc_k_gemm_bf16(0, None, 0, None, None, None, 0, 1, 1, 64, -1, None) == -1
    assert L.aenc_k_copy(None, None, 16, None) == -1
    assert L.aenc_k_copy_stream(None, None, 16, None) == -1
    assert L.aenc_k_mfma_loop(None, 1, 1, None, None) == -1
    assert L.aenc_k_mfma_loop(ctypes.c_void_p(16), 0, 1, None, None) == -1
    assert L.aenc_k_mfma_loop(ctypes.c_void_p(16), 1, 1, ctypes.c_void_p(12), None) == -1
    assert L.aenc_k_row_stream(None, None, 1, 1280, None) == -1
    assert L.aenc_k_row_stream(ctypes.c_void_p(16), ctypes.c_void_p(16), 1, 1282, None) == -1
    assert L.aenc_k_row_stream(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, 1280, None) == -1
    assert L.aenc_k_row_stream(ctypes.c_void_p(8), ctypes.c_void_p(16), 1, 1280, None) == -1
    # kernel entry points reject bad sizes before any launch
    buf = ctypes.c_void_p(16)
    assert L.aenc_k_gemm_bf16(0, buf, 64, buf, None, buf, 64, 64, 64, 100, -1, None) == -1
    assert L.aenc_k_layernorm(buf, buf, buf, buf, 0, 4, 4096, 1e-5, None) == -1
    # ... and operands not 16-byte aligned (the kernels move 16 bytes per lane)
    odd = ctypes.c_void_p(24)
    assert L.aenc_k_gemm_bf16(0, buf, 64, buf, None, odd, 64, 64, 64, 64, -1, None) == -1
    assert "aligned" in aenc.last_error()
    assert L.aenc_k_gemm_bf16(0, odd, 64, buf, None, buf, 64, 64, 64, 64, -1, None) == -1
    assert L.aenc_k_qkv_bf16(buf, buf, odd, ctypes.c_float(1.0), buf, buf, 128, 64, 64, None) == -1
    assert "aligned" in aenc.last_error()
    i32 = ctypes.c_void_p(64)
    assert L.aenc_k_attention_bf16(buf, buf, 64, i32, i32, 1, 8, 1, None, None, odd, None) == -1
    assert "aligned" in aenc.last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the path taken when no device exists")
def test_create_without_device_reports_it(aenc):
    w = synth.get_workload("tiny_fp32_b1")
    W = {k: torch.from_numpy(v) for k, v in synth.make_weights(w).items()}
    with pytest.raises(aenc.AencError, match="no HIP device"):
        aenc.Encoder(w.geom, W)


def test_cache_content_keys(aenc):
    """key_of: deterministic, sensitive to one changed value, to dtype and to shape."""
    import numpy as np
    a = np.arange(4800, dtype=np.float32)
    k = aenc.EmbeddingsCache.key_of(a)
    assert k == aenc.EmbeddingsCache.key_of(a.copy()) == aenc.EmbeddingsCache.key_of(torch.from_numpy(a))
    assert 0 <= k < 2 ** 64
    b = a.copy()
    b[1234] += 1.0
    assert aenc.EmbeddingsCache.key_of(b) != k
    assert aenc.EmbeddingsCache.key_of(a.reshape(48, 100)) != k
    assert aenc.EmbeddingsCache.key_of(a.view(np.int32)) != k
    bf = torch.from_numpy(a).to(torch.bfloat16)
    assert aenc.EmbeddingsCache.key_of(bf) == aenc.EmbeddingsCache.key_of(bf.clone())
    assert aenc.EmbeddingsCache.key_of(bf) != aenc.EmbeddingsCache.key_of(bf.view(torch.int16))


def test_chunked_attention_geometry(aenc):
    g = synth.get_workload("whisper_medium_pool2_chunk1s_b16").geom
    assert aenc.validate(g) == 0
    assert aenc.output_shape(g) == (16, 750, 1024)
    # the chunk rule changes no parameter and no shape
    assert aenc.param_count(g) == aenc.param_count(g.replace(attn_chunk=0, attn_chunk_mode=0))
    for bad in (dict(attn_chunk=-1), dict(attn_chunk=1501), dict(attn_chunk=50, attn_chunk_mode=0),
                dict(attn_chunk=50, attn_chunk_mode=3), dict(attn_chunk=0, attn_chunk_mode=1)):
        assert aenc.validate(g.replace(**bad)) == -1, bad
        assert "attn_chunk" in aenc.last_error()
    assert aenc.validate(g.replace(attn_chunk=1500, attn_chunk_mode=2)) == 0
    # the workspace holds two more int32 per packed row and copy
    assert aenc.lib().aenc_workspace_bytes(ctypes.byref(aenc._lib.geometry(g))) > \
        aenc.lib().aenc_workspace_bytes(ctypes.byref(aenc._lib.geometry(g.replace(attn_chunk=0, attn_chunk_mode=0))))


def test_chunk_step_rejects_bad_arguments(aenc):
    L = aenc.lib()
    p = ctypes.c_void_p(16)      # never dereferenced: every call fails its host checks
    assert L.aenc_k_chunk_ranges(None, 1, 10, 5, 1, None, p, p, p, None) == -1
    assert L.aenc_k_chunk_ranges(None, 1, 10, 0, 1, p, p, p, p, None) == -1
    assert L.aenc_k_chunk_ranges(None, 1, 10, 5, 3, p, p, p, p, None) == -1
    assert L.aenc_k_chunk_ranges(None, 1, 5000, 5, 1, p, p, p, p, None) == -1
    assert L.aenc_k_attention_bf16(p, p, 64, p, p, 1, 10, 1, p, None, p, None) == -1
    assert "together" in aenc.last_error()
