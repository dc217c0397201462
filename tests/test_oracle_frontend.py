"""Pins of the log-mel front-end oracle (oracle/frontend.py).

The pages name a Whisper feature extractor and fix its geometry (16 kHz,
480,000 samples per 30 s chunk, n_fft 400, hop 160, 128 features, 3000
frames); the `transformers` WhisperFeatureExtractor, an independent
implementation of that extractor, pins every step of the oracle, and a
textbook DFT loop pins the spectrum on its own. Plausible mistakes planted in
the oracle must each fail a pin.
"""
import math

import numpy as np
import pytest

import synth
from oracle import frontend as FE

transformers = pytest.importorskip("transformers")


def whisper_extractor(n_mels):
    from transformers import WhisperFeatureExtractor
    return WhisperFeatureExtractor(feature_size=n_mels, sampling_rate=16000, hop_length=160, chunk_length=30,
                                   n_fft=400)


@pytest.fixture(scope="module")
def clips():
    return synth.make_audio(11, 2)


def library_features(x, n_mels):
    return whisper_extractor(n_mels)(x, sampling_rate=16000, return_tensors="np")["input_features"][0]


def pins_pass(clips) -> bool:
    try:
        for n_mels in (128, 80):
            got = FE.log_mel(clips[0], n_mels)
            ref = library_features(clips[0], n_mels)
            if got.shape != ref.shape or not np.allclose(got, ref, rtol=0, atol=1e-4):
                return False
    except Exception:
        return False
    return True


def test_frame_count_is_the_pages(page_facts):
    f = page_facts["feature_frames"]
    n = f["chunk_seconds"] * f["sampling_rate"]
    assert FE.power_spectrum(np.zeros(n), f["n_fft"], f["hop_length"]).shape == (f["n_fft"] // 2 + 1,
                                                                                 f["nb_max_frames"])


@pytest.mark.parametrize("n_mels", [128, 80])
def test_log_mel_matches_the_whisper_extractor(clips, n_mels):
    for x in clips:
        got = FE.log_mel(x, n_mels)
        ref = library_features(x, n_mels)
        assert got.shape == ref.shape == (n_mels, 3000)
        # the library rounds to float32 after the spectrum: deep spectral valleys
        # differ by up to ~3e-5 (the median element by 4e-8)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-4)


def test_filters_match_the_library():
    from transformers.audio_utils import mel_filter_bank
    ref = mel_filter_bank(num_frequency_bins=201, num_mel_filters=128, min_frequency=0.0, max_frequency=8000.0,
                          sampling_rate=16000, norm="slaney", mel_scale="slaney")
    np.testing.assert_allclose(FE.mel_filters(128), ref.T, rtol=1e-10, atol=1e-14)


def test_power_spectrum_by_a_textbook_dft():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1200)
    got = FE.power_spectrum(x)
    pad = np.concatenate([x[200:0:-1], x, x[-2:-202:-1]])     # reflect by 200 on both sides
    w = [0.5 - 0.5 * math.cos(2 * math.pi * i / 400) for i in range(400)]
    n_frames = 1200 // 160
    assert got.shape == (201, n_frames)
    for f in range(n_frames):
        seg = pad[160 * f:160 * f + 400]
        for k in (0, 1, 37, 100, 200):
            re = sum(w[n] * seg[n] * math.cos(2 * math.pi * k * n / 400) for n in range(400))
            im = -sum(w[n] * seg[n] * math.sin(2 * math.pi * k * n / 400) for n in range(400))
            assert got[k, f] == pytest.approx(re * re + im * im, rel=1e-9, abs=1e-9)


def test_mel_scale_is_continuous_at_1khz_and_invertible():
    f = np.linspace(0, 8000, 1001)
    np.testing.assert_allclose(FE.mel_to_hz(FE.hz_to_mel(f)), f, rtol=1e-12, atol=1e-9)
    assert FE.hz_to_mel(1000.0) == pytest.approx(15.0, abs=1e-12)
    assert FE.hz_to_mel(999.999999) == pytest.approx(FE.hz_to_mel(1000.0), abs=1e-6)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
REAL = {n: getattr(FE, n) for n in ("hann_periodic", "frames", "hz_to_mel", "mel_to_hz", "mel_filters",
                                     "power_spectrum", "log_mel")}


def m_symmetric_hann(n):
    i = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * math.pi * i / (n - 1))


def m_zero_pad_frames(x, n_fft=FE.N_FFT, hop=FE.HOP):
    xp = np.pad(np.asarray(x, np.float64), n_fft // 2)
    n = 1 + (len(xp) - n_fft) // hop
    return np.stack([xp[hop * f: hop * f + n_fft] for f in range(n)])


def m_htk_hz_to_mel(f):
    return 2595.0 * np.log10(1.0 + np.asarray(f, np.float64) / 700.0)


def m_htk_mel_to_hz(m):
    return 700.0 * (10.0 ** (np.asarray(m, np.float64) / 2595.0) - 1.0)


def m_unnormalised_filters(n_mels, n_fft=FE.N_FFT, sample_rate=FE.SAMPLE_RATE):
    fb = REAL["mel_filters"](n_mels, n_fft, sample_rate)
    return fb / fb.max(axis=1, keepdims=True)


def m_magnitude_not_power(x, n_fft=FE.N_FFT, hop=FE.HOP):
    return np.sqrt(REAL["power_spectrum"](x, n_fft, hop))


def m_natural_log(x, n_mels=128, n_fft=FE.N_FFT, hop=FE.HOP, sample_rate=FE.SAMPLE_RATE):
    mel = FE.mel_filters(n_mels, n_fft, sample_rate) @ FE.power_spectrum(x, n_fft, hop)
    lg = np.log(np.maximum(mel, 1e-10))
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0


def m_no_range_floor(x, n_mels=128, n_fft=FE.N_FFT, hop=FE.HOP, sample_rate=FE.SAMPLE_RATE):
    mel = FE.mel_filters(n_mels, n_fft, sample_rate) @ FE.power_spectrum(x, n_fft, hop)
    return (np.log10(np.maximum(mel, 1e-10)) + 4.0) / 4.0


def m_keeps_last_frame(x, n_fft=FE.N_FFT, hop=FE.HOP):
    fr = REAL["frames"](x, n_fft, hop) * FE.hann_periodic(n_fft)[None, :]
    return (np.abs(np.fft.rfft(fr, axis=1)) ** 2).T


MUTATIONS = {
    "symmetric_hann": ("hann_periodic", m_symmetric_hann),
    "zero_padded_frames": ("frames", m_zero_pad_frames),
    "htk_mel_scale": (("hz_to_mel", "mel_to_hz"), (m_htk_hz_to_mel, m_htk_mel_to_hz)),
    "filters_not_area_normalised": ("mel_filters", m_unnormalised_filters),
    "magnitude_not_power": ("power_spectrum", m_magnitude_not_power),
    "natural_log": ("log_mel", m_natural_log),
    "no_80db_floor": ("log_mel", m_no_range_floor),
    "last_frame_kept": ("power_spectrum", m_keeps_last_frame),
}


def test_unmutated_frontend_passes(clips):
    assert pins_pass(clips)


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_frontend_mistake_is_caught(clips, mutation, monkeypatch):
    names, fns = MUTATIONS[mutation]
    if isinstance(names, str):
        names, fns = (names,), (fns,)
    for n, f in zip(names, fns):
        monkeypatch.setattr(FE, n, f)
    assert not pins_pass(clips), f"planted mistake {mutation!r} was not caught"
