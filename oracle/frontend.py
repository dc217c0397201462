"""Reference log-mel front end (test infrastructure only), float64 NumPy.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline may import
this module; the library never does.

The pages fix the feature extractor's geometry: a Whisper feature extractor
with 16 kHz audio, 30 s chunks of 480,000 samples, n_fft 400, hop 160, 128
features and at most 3000 frames ("Voxtral-Mini-3B-2507", Preprocessor;
"Qwen2-Audio-7B-Instruct" uses the same Whisper front end). They name the
extractor but do not spell out its steps, so this module takes the Whisper
extractor's published recipe as the reading, step by step:

  1. centred frames: the signal is reflect-padded by n_fft/2 on both sides and
     frame f covers padded samples [hop f, hop f + n_fft);
  2. a periodic Hann window, w[i] = 1/2 - 1/2 cos(2 pi i / n_fft);
  3. the power spectrum |DFT|^2 of each frame, bins 0 .. n_fft/2; the last
     frame is dropped, so 480,000 samples give exactly 3000 frames;
  4. a bank of triangular mel filters on the Slaney mel scale (linear below
     1 kHz, logarithmic above), 0 Hz to the Nyquist frequency, each filter
     scaled to unit area (Slaney normalisation);
  5. log10 of the filter outputs floored at 1e-10, then floored again at the
     clip's maximum minus 8 (an 80 dB range), then (x + 4) / 4.

The whole recipe is pinned against the `transformers` WhisperFeatureExtractor
in tests/test_oracle_frontend.py; the DFT also against a textbook loop.
"""
from __future__ import annotations

import math

import numpy as np

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160


def hann_periodic(n: int) -> np.ndarray:
    """w[i] = 1/2 - 1/2 cos(2 pi i / n), i < n (the periodic Hann window)."""
    i = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * math.pi * i / n)


def frames(x: np.ndarray, n_fft: int = N_FFT, hop: int = HOP) -> np.ndarray:
    """Centred frames [n_frames, n_fft] of a 1-D signal: reflect padding of
    n_fft/2 on both sides, frame f starts at padded sample hop f."""
    pad = n_fft // 2
    xp = np.pad(np.asarray(x, np.float64), pad, mode="reflect")
    n = 1 + (len(xp) - n_fft) // hop
    return np.stack([xp[hop * f: hop * f + n_fft] for f in range(n)])


def power_spectrum(x: np.ndarray, n_fft: int = N_FFT, hop: int = HOP) -> np.ndarray:
    """|DFT(window * frame)|^2 for bins 0 .. n_fft/2: [n_fft/2 + 1, n_frames - 1]
    (the last centred frame is dropped)."""
    fr = frames(x, n_fft, hop) * hann_periodic(n_fft)[None, :]
    spec = np.fft.rfft(fr, axis=1)                  # library DFT, bins 0 .. n_fft/2
    return (np.abs(spec) ** 2).T[:, :-1]


def hz_to_mel(f):
    """Slaney mel scale: 3 f / 200 below 1 kHz, then 15 + 27 ln(f / 1000) / ln 6.4."""
    f = np.asarray(f, np.float64)
    lin = 3.0 * f / 200.0
    log = 15.0 + 27.0 * np.log(np.maximum(f, 1e-12) / 1000.0) / math.log(6.4)
    return np.where(f >= 1000.0, log, lin)


def mel_to_hz(m):
    m = np.asarray(m, np.float64)
    lin = 200.0 * m / 3.0
    log = 1000.0 * np.exp((m - 15.0) * math.log(6.4) / 27.0)
    return np.where(m >= 15.0, log, lin)


def mel_filters(n_mels: int, n_fft: int = N_FFT, sample_rate: int = SAMPLE_RATE) -> np.ndarray:
    """Triangular filters [n_mels, n_fft/2 + 1] with edges evenly spaced in mel
    between 0 Hz and sample_rate / 2, each scaled by 2 / (upper - lower edge in Hz)."""
    n_bins = n_fft // 2 + 1
    freqs = np.linspace(0.0, sample_rate / 2.0, n_bins)
    edges = mel_to_hz(np.linspace(hz_to_mel(0.0), hz_to_mel(sample_rate / 2.0), n_mels + 2))
    fb = np.zeros((n_mels, n_bins))
    for m in range(n_mels):
        lo, mid, hi = edges[m], edges[m + 1], edges[m + 2]
        rise = (freqs - lo) / (mid - lo)
        fall = (hi - freqs) / (hi - mid)
        fb[m] = np.maximum(0.0, np.minimum(rise, fall)) * (2.0 / (hi - lo))
    return fb


def log_mel(x: np.ndarray, n_mels: int = 128, n_fft: int = N_FFT, hop: int = HOP,
            sample_rate: int = SAMPLE_RATE) -> np.ndarray:
    """One clip: samples [n] -> features [n_mels, n / hop]."""
    mel = mel_filters(n_mels, n_fft, sample_rate) @ power_spectrum(x, n_fft, hop)
    lg = np.log10(np.maximum(mel, 1e-10))
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0


def log_mel_batch(audio: np.ndarray, n_mels: int = 128) -> np.ndarray:
    """[B, n] -> [B, n_mels, n / hop]; clips are independent."""
    return np.stack([log_mel(a, n_mels) for a in audio])
