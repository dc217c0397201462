"""aenc_forward_noalloc: the forward with its activations in the library's
static scratch array instead of the handle's workspace, for callers that
cannot allocate. Checked through the C ABI against aenc_forward on the same
inputs (the bf16 bar, and bit for bit: the same kernels on the same data) on
two calls in a row, the second with fewer clips, and against the oracle."""
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


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _encoder(aenc, w, W):
    return aenc.Encoder(w.geom, {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for k, v in W.items()})


def _noalloc(aenc, enc, n_clips, mel, mask, out):
    st = aenc.lib().aenc_forward_noalloc(enc._h, n_clips, _p(mel), _p(mask), _p(out), _stream())
    assert st == 0, aenc.last_error()


def test_noalloc_matches_the_forward_on_two_calls(aenc):
    # Whisper-large width, 2 blocks, 3 clips of 500 positions, the last two masked short
    base = synth.get_workload("whisper_large_b1")
    w = base.replace(geom=base.geom.replace(batch=3, n_layers=2, n_frames=1000), init="perturbed")
    g = w.geom
    W = synth.make_weights(w)
    mel_np = synth.make_mel(w)
    n_f = np.array([1000, 613, 141])
    for b, n in enumerate(n_f):
        mel_np[b, :, n:] = 0.0
    mask_np = (np.arange(g.n_pos)[None, :] < ((n_f + 1) // 2)[:, None]).astype(np.uint8)
    need3 = aenc.lib().aenc_noalloc_scratch_bytes(ctypes.byref(aenc._lib.geometry(g)), 3)
    assert 0 < need3 <= aenc._lib.AENC_NOALLOC_SCRATCH_BYTES
    enc = _encoder(aenc, w, W)
    mel = torch.from_numpy(mel_np).to(DEV).to(torch.bfloat16)
    mask = torch.from_numpy(mask_np).to(DEV)
    ref = enc.forward(mel, mask).clone()
    torch.cuda.synchronize()
    valid = mask_np.astype(bool)
    want = oracle.encode(g, W, mel_np, mask_np)

    # call 1: all three clips, masked
    out1 = torch.full(enc.out_shape, float("nan"), device=DEV, dtype=enc.out_dtype)
    print("noalloc call 1: 3 clips, masked", flush=True)
    _noalloc(aenc, enc, 3, mel, mask, out1)
    torch.cuda.synchronize()
    got1 = out1.double().cpu().numpy()
    m = parity.assert_bf16_parity(got1[valid], ref.double().cpu().numpy()[valid], "noalloc call 1 vs forward")
    print("call 1 vs forward", m, "bitwise", torch.equal(out1, ref), flush=True)
    assert np.all(got1[~valid] == 0.0)
    parity.assert_bf16_parity(got1[valid], want[valid], "noalloc call 1 vs oracle")

    # call 2: one clip (a smaller input), no mask, against a batch-1 handle's forward
    w1 = w.replace(geom=g.replace(batch=1))
    enc1 = _encoder(aenc, w1, W)
    mel1 = mel[:1].contiguous()
    ref1 = enc1.forward(mel1).clone()
    out2 = torch.full((1,) + tuple(enc.out_shape[1:]), float("nan"), device=DEV, dtype=enc.out_dtype)
    print("noalloc call 2: 1 clip", flush=True)
    _noalloc(aenc, enc, 1, mel1, None, out2)
    torch.cuda.synchronize()
    m = parity.assert_bf16_parity(out2.double().cpu().numpy()[0], ref1.double().cpu().numpy()[0],
                                  "noalloc call 2 vs forward")
    print("call 2 vs forward", m, "bitwise", torch.equal(out2, ref1), flush=True)
    parity.assert_bf16_parity(out2.double().cpu().numpy()[0], oracle.encode(g, W, mel_np[:1])[0],
                              "noalloc call 2 vs oracle")
    enc1.close()
    enc.close()


def test_noalloc_rejects_what_does_not_fit(aenc):
    w = synth.get_workload("whisper_large_b1")
    g = w.geom.replace(batch=3, n_layers=1)
    cg = ctypes.byref(aenc._lib.geometry(g))
    L = aenc.lib()
    need = [L.aenc_noalloc_scratch_bytes(cg, n) for n in (1, 2, 3)]
    assert 0 < need[0] <= aenc._lib.AENC_NOALLOC_SCRATCH_BYTES < need[1] < need[2]
    assert L.aenc_noalloc_scratch_bytes(cg, 0) == -1 and L.aenc_noalloc_scratch_bytes(cg, 4) == -1
    W = synth.make_weights(w.replace(geom=g))
    enc = _encoder(aenc, w.replace(geom=g), W)
    mel = torch.zeros(3, g.n_mel, g.n_frames, device=DEV, dtype=torch.bfloat16)
    out = torch.zeros(enc.out_shape, device=DEV, dtype=enc.out_dtype)
    assert L.aenc_forward_noalloc(enc._h, 2, _p(mel), None, _p(out), _stream()) == -1
    assert "scratch" in aenc.last_error()
    assert L.aenc_forward_noalloc(enc._h, 4, _p(mel), None, _p(out), _stream()) == -1
    assert L.aenc_forward_noalloc(enc._h, 0, _p(mel), None, _p(out), _stream()) == -1
    assert L.aenc_forward_noalloc(None, 1, _p(mel), None, _p(out), _stream()) == -1
    assert L.aenc_forward_noalloc(enc._h, 1, None, None, _p(out), _stream()) == -1
    _noalloc(aenc, enc, 1, mel, None, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0]).all()
    enc.close()
