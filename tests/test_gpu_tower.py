"""End-to-end parity of the HIP tower (through include/aenc.h) with the oracle.

Reduced geometries are compared element by element on every row; the five
full-size workloads are compared on sampled clips (each run alone by the
oracle, clips being independent) and, for the larger ones, sampled rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def aenc():
    import audio_encoder_tower_amd as a
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    a.lib()
    return a


def device_weights(W, dtype):
    tdt = torch.bfloat16 if dtype == synth.workloads.BF16 else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV).to(tdt) for k, v in W.items()}


def run_gpu(aenc, w, W=None, mel=None, mask=None, clips=None):
    g = w.geom
    if W is None:
        W = synth.make_weights(w)
    if mel is None:
        mel = synth.make_mel(w, clips=clips)
        mask = synth.make_mask(w, clips=clips)
    print(f"gpu forward {w.name} geom={g}", flush=True)
    enc = aenc.Encoder(g, device_weights(W, g.dtype))
    tdt = torch.bfloat16 if g.dtype == synth.workloads.BF16 else torch.float32
    mel_d = torch.from_numpy(mel).to(DEV).to(tdt)
    mask_d = None if mask is None else torch.from_numpy(mask).to(DEV)
    out = enc.forward(mel_d, mask_d)
    torch.cuda.synchronize()
    res = out.float().cpu().numpy().astype(np.float64)
    enc.close()
    return res


def tiny(name="tiny_fp32_b1", **kw):
    w = synth.get_workload(name)
    return w.replace(geom=w.geom.replace(**kw))


def reduced(base, name, geom_kw, **wkw):
    w = synth.get_workload(base)
    return w.replace(name=name, geom=w.geom.replace(**geom_kw), **wkw)


REDUCED = {
    # Whisper-large width, 2 blocks, 700 positions (ragged against 64/128/256 tiles), 2 clips
    "large_width_ragged": reduced("whisper_large_b1", "large_width_ragged",
                                  dict(n_layers=2, n_frames=1400, batch=2), init="perturbed"),
    # Whisper-medium width with the pool over an odd number of positions
    "medium_pool_odd": reduced("whisper_medium_pool2_b1", "medium_pool_odd",
                               dict(n_layers=2, n_frames=802), init="perturbed"),
    # projector with a key mask over 3 clips
    "projector_masked": reduced("whisper_large_b1", "projector_masked",
                                dict(batch=3, n_layers=1, n_frames=900, d_model=256, n_heads=4, d_ffn=1024,
                                     proj_hidden=512, proj_out=384), init="perturbed"),
    # full-width variable-length batch, one block
    "varlen_large_1block": reduced("whisper_large_varlen_b32", "varlen_large_1block",
                                   dict(batch=4, n_layers=1)),
    # sharp attention (Q and K weights std 0.05: scores of std ~3)
    "sharp_attention": reduced("whisper_large_b1", "sharp_attention",
                               dict(n_layers=2, n_frames=600), init="sharp"),
    # no blocks: stem, positions and final LayerNorm only
    "no_blocks": reduced("whisper_large_b1", "no_blocks", dict(n_layers=0, batch=2), init="perturbed"),
    # bf16 output
    "bf16_out": reduced("whisper_large_b1", "bf16_out", dict(n_layers=1, n_frames=400, out_dtype="bf16"),
                        init="perturbed"),
    # the tiny fp32 geometry with nonzero biases and a mask
    "fp32_perturbed_masked": reduced("tiny_fp32_b1", "fp32_perturbed_masked", dict(batch=3), init="perturbed"),
    "fp32_projector": reduced("tiny_fp32_b1", "fp32_projector", dict(proj_hidden=128, proj_out=192),
                              init="perturbed"),
    # 4 positions stacked into the projector input, key mask over 3 clips
    "stack4_masked": reduced("whisper_large_b1", "stack4_masked",
                             dict(batch=3, n_layers=1, n_frames=900, d_model=256, n_heads=4, d_ffn=1024,
                                  proj_hidden=512, proj_out=384, stack=4), init="perturbed"),
    # Whisper-large width, stacked 5120-wide projector input, 2 clips of 500 positions
    "stack4_large_width": reduced("whisper_large_b1", "stack4_large_width",
                                  dict(batch=2, n_layers=1, n_frames=1000, proj_hidden=3072, proj_out=3072,
                                       stack=4), init="perturbed"),
    "fp32_stack4": reduced("tiny_fp32_b1", "fp32_stack4", dict(proj_hidden=128, proj_out=192, stack=4, batch=2),
                           init="perturbed"),
    # chunked attention (1 s = 50 positions), chunk-causal, Whisper-medium width, pool 2, key mask over 3 clips
    "chunk_causal_masked": reduced("whisper_medium_pool2_chunk1s_b16", "chunk_causal_masked",
                                   dict(batch=3, n_layers=2, n_frames=900), init="perturbed"),
    # block-diagonal chunks that do not divide the clip, ragged against the 128-query tiles
    "chunk_block_ragged": reduced("whisper_large_b1", "chunk_block_ragged",
                                  dict(batch=2, n_layers=2, n_frames=700, attn_chunk=37, attn_chunk_mode=2),
                                  init="perturbed"),
    # chunk of one position: block-diagonal attention returns each position's values
    "chunk_block_one": reduced("whisper_large_b1", "chunk_block_one",
                               dict(n_layers=1, n_frames=300, attn_chunk=1, attn_chunk_mode=2), init="perturbed"),
    # chunk of one position, causal: ordinary causal attention
    "chunk_causal_one": reduced("whisper_large_b1", "chunk_causal_one",
                                dict(n_layers=1, n_frames=300, attn_chunk=1, attn_chunk_mode=1), init="sharp"),
    # the fp32 path with chunk-causal attention and a key mask
    "fp32_chunk_causal_masked": reduced("tiny_fp32_b1", "fp32_chunk_causal_masked",
                                        dict(batch=3, attn_chunk=16, attn_chunk_mode=1), init="perturbed"),
    "fp32_chunk_block": reduced("tiny_fp32_b1", "fp32_chunk_block", dict(attn_chunk=30, attn_chunk_mode=2),
                                init="perturbed"),
    # a clip with no valid position at all (its rows come out as zeros), with the projector
    "empty_clip_masked": reduced("whisper_large_b1", "empty_clip_masked",
                                 dict(batch=3, n_layers=1, n_frames=400, d_model=256, n_heads=4, d_ffn=1024,
                                      proj_hidden=512, proj_out=384), init="perturbed"),
    # degenerate sizes: two mel frames -> one position; four frames pooled into one output row
    "one_position": reduced("whisper_large_b1", "one_position", dict(batch=3, n_layers=2, n_frames=2),
                            init="perturbed"),
    "pool_one_output": reduced("whisper_medium_pool2_b1", "pool_one_output", dict(batch=2, n_layers=1, n_frames=4),
                               init="perturbed"),
    "projector_one_position": reduced("whisper_large_b1", "projector_one_position",
                                      dict(n_layers=1, n_frames=2, proj_hidden=3072, proj_out=3072),
                                      init="perturbed"),
    # a long masked batch on the 256x256 tiles: the device row count (12 clips, several short) leaves
    # 190 tiles of valid rows of the 355 the launch is sized for, split evenly over the XCDs
    "batch12_masked": reduced("whisper_large_b1", "batch12_masked", dict(batch=12, n_layers=1), init="perturbed"),
}


# Explicit valid mel frames per clip for some reduced cases (frames past them
# are zeroed, positions past ceil(n_f / 2) masked).
LENGTHS = {
    "projector_masked": [900, 411, 101],
    "fp32_perturbed_masked": [200, 137, 61],
    "stack4_masked": [900, 411, 101],
    "fp32_stack4": [200, 117],
    "chunk_causal_masked": [900, 433, 97],
    "empty_clip_masked": [400, 0, 51],
    "fp32_chunk_causal_masked": [200, 137, 61],
    "batch12_masked": [3000, 2999, 1700, 900, 401, 3000, 100, 2000, 1200, 800, 3000, 57],
}


def inputs(w):
    mel = synth.make_mel(w)
    mask = synth.make_mask(w)
    if w.name in LENGTHS:
        n_f = np.array(LENGTHS[w.name])
        for b, n in enumerate(n_f):
            mel[b, :, n:] = 0.0
        mask = (np.arange(w.geom.n_pos)[None, :] < ((n_f + 1) // 2)[:, None]).astype(np.uint8)
    return mel, mask


def compare(w, got, ref, mask, what):
    g = w.geom
    rows = np.ones(got.shape[:2], bool)
    if mask is not None:
        # an output row is defined when every position it reads is valid
        t_out, span = g.t_out, g.pool_step * g.stack
        valid = mask[:, : t_out * span].reshape(mask.shape[0], t_out, span).all(-1)
        rows = valid
        # masked rows are written as zeros
        assert np.all(got[~rows] == 0.0), f"{what}: masked rows not zero"
    if g.dtype == synth.workloads.F32 and g.out_dtype == synth.workloads.F32:
        return parity.assert_f32_parity(got[rows], ref[rows], what)
    return parity.assert_bf16_parity(got[rows], ref[rows], what)


@pytest.mark.parametrize("case", sorted(REDUCED))
def test_reduced_tower(aenc, case):
    w = REDUCED[case]
    W = synth.make_weights(w)
    mel, mask = inputs(w)
    got = run_gpu(aenc, w, W, mel, mask)
    ref = oracle.encode(w.geom, W, mel, mask)
    assert got.shape == ref.shape == (w.geom.batch, w.geom.t_out, w.geom.d_out)
    m = compare(w, got, ref, mask, case)
    print(case, m)


@pytest.mark.parametrize("name", list(parity.FULL_SIZE_SAMPLES))
def test_full_size_workload(aenc, name):
    w = synth.get_workload(name)
    g = w.geom
    W = synth.make_weights(w)
    mel = synth.make_mel(w)
    mask = synth.make_mask(w)
    got = run_gpu(aenc, w, W, mel, mask)
    assert got.shape == (g.batch, g.t_out, g.d_out)
    assert np.isfinite(got).all()
    every = parity.FULL_SIZE_SAMPLES[name]["every"]
    for clip in parity.full_size_clips(w):
        ref = parity.oracle_clip(w, clip, W, every=every)
        rows = ref["rows"]
        g_rows = got[clip][rows]
        clip_mask = None
        if mask is not None:
            valid = mask[clip][rows].astype(bool)
            assert np.all(g_rows[~valid] == 0.0)
            g_rows, r_rows = g_rows[valid], ref["out"][valid]
        else:
            r_rows = ref["out"]
        if g.dtype == synth.workloads.F32:
            m = parity.assert_f32_parity(g_rows, r_rows, f"{name} clip {clip}")
        else:
            m = parity.assert_bf16_parity(g_rows, r_rows, f"{name} clip {clip}")
        print(name, clip, m, flush=True)


def test_deterministic_and_batch_independent(aenc):
    w = reduced("whisper_large_varlen_b32", "det", dict(batch=3, n_layers=2, n_frames=1000), init="perturbed")
    W = synth.make_weights(w)
    mel = synth.make_mel(w)
    mask = synth.make_mask(w)
    a = run_gpu(aenc, w, W, mel, mask)
    b = run_gpu(aenc, w, W, mel, mask)
    np.testing.assert_array_equal(a, b)
    one = w.replace(geom=w.geom.replace(batch=1))
    c = run_gpu(aenc, one, W, mel[1:2], mask[1:2])
    np.testing.assert_array_equal(a[1], c[0])


def test_forward_at_the_bf16_batch_limit(aenc):
    """The largest Whisper-large bf16 batch that validation accepts (278
    clips): the FFN hidden rows then span 4,281,466,880 bytes, so the GEMM
    copies of the last clips use buffer offsets above 2^31. Clips 0..275 hold
    one mel (stream 0) and must come out bit-identical to each other; the last
    two clips hold mels of their own (streams 1 and 2), so that a wrong offset
    above 2^31 that read another clip's rows could not pass, and each is
    checked against its own oracle output."""
    w = synth.get_workload("whisper_large_b1")
    W = synth.make_weights(w)
    g = w.geom.replace(batch=278)
    assert aenc.validate(g) == 0 and aenc.validate(g.replace(batch=279)) == -1
    print(f"gpu forward whisper_large_b1 x 278 geom={g}", flush=True)
    enc = aenc.Encoder(g, device_weights(W, g.dtype))
    mels = torch.from_numpy(synth.make_mel(w, clips=[0, 1, 2])).to(DEV).to(torch.bfloat16)
    mel = mels[0:1].expand(g.batch, -1, -1).contiguous()
    mel[276] = mels[1]
    mel[277] = mels[2]
    out = enc.forward(mel)
    torch.cuda.synchronize()
    picks = [0, 139, 275, 276, 277]
    got = out[picks].float().cpu().numpy().astype(np.float64)
    del out, mel
    enc.close()
    for i in (1, 2):
        np.testing.assert_array_equal(got[i], got[0], err_msg=f"clip {picks[i]} differs from clip 0")
    for i, stream in ((0, 0), (3, 1), (4, 2)):
        ref = parity.oracle_clip(w, stream, W, every=1)
        m = parity.assert_bf16_parity(got[i][ref["rows"]], ref["out"], f"batch 278, clip {picks[i]}")
        print(f"batch limit clip {picks[i]} (mel stream {stream})", m, flush=True)


def test_padded_frames_do_not_change_valid_rows(aenc):
    w = reduced("whisper_large_varlen_b32", "pad", dict(batch=2, n_layers=2, n_frames=1200), init="perturbed")
    W = synth.make_weights(w)
    mel = synth.make_mel(w)
    mask = synth.make_mask(w)
    base = run_gpu(aenc, w, W, mel, mask)
    junk = mel.copy()
    rng = np.random.default_rng(0)
    for b in range(w.geom.batch):
        tb = int(mask[b].sum())
        junk[b, :, 2 * tb + 1:] = synth.round_to_bf16(
            rng.choice([-1e4, 1e4], size=junk[b, :, 2 * tb + 1:].shape).astype(np.float32))
    other = run_gpu(aenc, w, W, junk, mask)
    for b in range(w.geom.batch):
        tb = int(mask[b].sum())
        np.testing.assert_array_equal(other[b, :tb], base[b, :tb])


def test_profile_counts_every_launch(aenc):
    w = reduced("whisper_large_b1", "prof", dict(n_layers=2, n_frames=400))
    g = w.geom
    W = synth.make_weights(w)
    enc = aenc.Encoder(g, device_weights(W, g.dtype))
    mel = torch.from_numpy(synth.make_mel(w)).to(DEV).to(torch.bfloat16)
    enc.profile(True)
    for _ in range(3):
        enc.forward(mel)
    torch.cuda.synchronize()
    stats = enc.profile_read()
    enc.close()
    assert stats["fc1"][1] == 3 * g.n_layers and stats["attention"][1] == 3 * g.n_layers
    assert stats["layernorm"][1] == 3 * 2 * g.n_layers
    assert all(ms >= 0 for ms, _ in stats.values())


def test_forward_rejects_bad_arguments(aenc):
    w = reduced("whisper_large_b1", "args", dict(n_layers=0, n_frames=64))
    g = w.geom
    W = synth.make_weights(w)
    enc = aenc.Encoder(g, device_weights(W, g.dtype))
    with pytest.raises(ValueError):
        enc.forward(torch.zeros(1, g.n_mel, g.n_frames + 2, device=DEV, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        enc.forward(torch.zeros(1, g.n_mel, g.n_frames, device=DEV, dtype=torch.float32))
    st = aenc.lib().aenc_forward(enc._h, None, None, None, None)
    assert st == -1 and "NULL" in aenc.last_error()
    # misaligned device pointers are refused before anything is enqueued
    mel = torch.zeros(1 * g.n_mel * g.n_frames + 8, device=DEV, dtype=torch.bfloat16)
    out = torch.zeros(1 << 20, device=DEV, dtype=torch.float32)
    st = aenc.lib().aenc_forward(enc._h, ctypes.c_void_p(mel.data_ptr() + 2), None,
                                 ctypes.c_void_p(out.data_ptr()), None)
    assert st == -1 and "aligned" in aenc.last_error()
    st = aenc.lib().aenc_forward(enc._h, ctypes.c_void_p(mel.data_ptr()), None,
                                 ctypes.c_void_p(out.data_ptr() + 4), None)
    assert st == -1 and "aligned" in aenc.last_error()
    enc.close()


@pytest.mark.parametrize("masked", [False, True], ids=["dense", "masked"])
def test_forward_in_hip_graph(aenc, masked):
    """aenc_forward enqueues without allocating or synchronising, so it can be
    captured into a HIP graph. Every replay (with eager forwards on the same
    handle in between) matches the eager result bit for bit."""
    w = reduced("whisper_large_b1", "graph", dict(n_layers=2, n_frames=400, batch=2), init="perturbed")
    g = w.geom
    enc = aenc.Encoder(g, device_weights(synth.make_weights(w), g.dtype))
    mel = torch.from_numpy(synth.make_mel(w)).to(DEV).to(torch.bfloat16)
    mask = None
    if masked:
        m = np.ones((g.batch, g.n_frames // 2), np.uint8)
        m[1, 130:] = 0
        mask = torch.from_numpy(m).to(DEV)
    ref = enc.forward(mel, mask).clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc.forward(mel, mask)                  # warm-up on a side stream, as torch asks before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    out = torch.empty_like(ref)
    with torch.cuda.graph(graph):
        enc.forward(mel, mask, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        eager = enc.forward(mel, mask)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)
    enc.close()
