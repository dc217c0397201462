"""GPU log-mel front end (aenc_frontend_*) against the fp64 front-end oracle."""
import ctypes
import numpy as np
import pytest
import torch

import synth
from oracle import frontend as FE

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def aenc():
    import audio_encoder_tower_amd as a
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    a.lib()
    return a


@pytest.mark.parametrize("n_samples,n_mel,clips", [(480000, 128, 2), (80000, 80, 3), (16000, 128, 1)],
                         ids=["30s_128", "5s_80", "1s_128"])
def test_frontend_matches_the_oracle(aenc, n_samples, n_mel, clips):
    audio = synth.make_audio(21, clips, n_samples)
    print(f"frontend {n_samples} samples, {n_mel} filters, {clips} clips", flush=True)
    fe = aenc.Frontend(clips, n_samples, n_mel, out_dtype="f32")
    got = fe(torch.from_numpy(audio).to(DEV))
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    fe.close()
    ref = FE.log_mel_batch(audio.astype(np.float64), n_mel)
    assert got.shape == ref.shape == (clips, n_mel, n_samples // 160)
    err = np.abs(got - ref)
    from tests import parity
    m = parity.assert_f32_parity(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]),
                                 f"frontend {n_samples}/{n_mel}")
    print(f"frontend {n_samples}/{n_mel}: max-abs {err.max():.3e}, median {np.median(err):.3e}, "
          f"normwise max-rel {m['max_rel']:.3e}", flush=True)
    # fp64 DFT sums: every feature within 1e-4 of the fp64 oracle, not only
    # relative to the largest one
    assert err.max() <= 1e-4, err.max()


def test_frontend_bf16_output_is_the_rounded_features(aenc):
    audio = synth.make_audio(22, 2, 160000)
    fe32 = aenc.Frontend(2, 160000, 128, out_dtype="f32")
    fe16 = aenc.Frontend(2, 160000, 128, out_dtype="bf16")
    x = torch.from_numpy(audio).to(DEV)
    a, b = fe32(x), fe16(x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(b.float().cpu().numpy(), a.to(torch.bfloat16).float().cpu().numpy())
    fe32.close()
    fe16.close()


def test_frontend_feeds_the_encoder(aenc):
    """Audio -> features -> tower on the GPU, checked against the oracle chain
    (features from the oracle front end, rounded to bf16, then the oracle tower)."""
    import oracle
    w = synth.get_workload("whisper_large_b1")
    w = w.replace(geom=w.geom.replace(n_layers=1, n_frames=1000, d_model=256, n_heads=4, d_ffn=1024), init="perturbed")
    g = w.geom
    audio = synth.make_audio(23, 1, g.n_frames * 160)
    fe = aenc.Frontend(1, g.n_frames * 160, g.n_mel, out_dtype="bf16")
    mel = fe(torch.from_numpy(audio).to(DEV))
    W = synth.make_weights(w)
    enc = aenc.Encoder(g, {k: torch.from_numpy(v).to(DEV).to(torch.bfloat16) for k, v in W.items()})
    out = enc.forward(mel)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    feats = synth.round_to_bf16(FE.log_mel_batch(audio.astype(np.float64), g.n_mel).astype(np.float32))
    # a GPU feature may sit on the other side of a bf16 rounding boundary than
    # the oracle's: compare the tower on the GPU's own features as well
    gpu_feats = mel.float().cpu().numpy()
    assert np.abs(gpu_feats - feats).max() <= 2.0 ** -7 * np.abs(feats).max()
    ref = oracle.encode(g, W, gpu_feats.astype(np.float32))
    from tests import parity
    parity.assert_bf16_parity(got[0], ref[0], "frontend -> tower")
    enc.close()
    fe.close()


def test_frontend_rejects_bad_arguments(aenc):
    with pytest.raises(Exception):
        aenc.Frontend(1, 1000, 128)          # not a multiple of 160
    fe = aenc.Frontend(1, 16000, 80)
    with pytest.raises(ValueError):
        fe(torch.zeros(1, 16160, device=DEV))
    assert aenc.lib().aenc_frontend_run(fe._h, None, None, None) == -1
    audio = torch.zeros(16000 + 8, device=DEV)
    mel = torch.zeros(80 * 100 + 8, device=DEV)
    assert aenc.lib().aenc_frontend_run(fe._h, ctypes.c_void_p(audio.data_ptr() + 4),
                                        ctypes.c_void_p(mel.data_ptr()), None) == -1
    assert "aligned" in aenc.last_error()
    fe.close()
