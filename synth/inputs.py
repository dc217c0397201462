"""Seeded synthetic weights, mel features, clip lengths and key masks.

Every tensor has its own random stream, spawned from a
``numpy.random.SeedSequence`` in the fixed order of ``weight_shapes``. So
adding the projector never changes the encoder weights, and clip ``i``'s mel
is the same whatever the batch size.

Values for a bf16 geometry are rounded to bf16 (round to nearest even) here,
once, and handed out as float32 arrays holding exactly representable bf16
values; both the oracle and the GPU path read those same values.

Weight matrices use the ``[out, in]`` convention of the checkpoints the
model records describe ("Qwen2-Audio-7B-Instruct", method note on reading
tensor shapes: q_proj.weight is [1280, 1280]); conv kernels are
``[out, in, 3]``. No key bias exists (the attention keys carry no bias).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

from .workloads import BF16, Geometry, Workload

LAYER_TENSORS = ("ln1_g", "ln1_b", "q_w", "q_b", "k_w", "v_w", "v_b", "o_w", "o_b",
                 "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")
PROJ_TENSORS = ("proj1_w", "proj1_b", "proj2_w", "proj2_b")
WEIGHT_STD = 0.02
# "sharp" init: query and key weights this wide give scores of standard
# deviation ~3 at d_model 1280 (peaked, but within what bf16 Q and K resolve;
# at 0.2 the rounding of Q and K to bf16 alone moves outputs by ~0.3).
SHARP_QK_STD = 0.05


def weight_shapes(g: Geometry) -> List[Tuple[str, Tuple[int, ...]]]:
    """Encoder tensors (projector excluded) in weights-struct order."""
    d, f = g.d_model, g.d_ffn
    out: List[Tuple[str, Tuple[int, ...]]] = [
        ("conv1_w", (d, g.n_mel, 3)), ("conv1_b", (d,)),
        ("conv2_w", (d, d, 3)), ("conv2_b", (d,)),
    ]
    per_layer = {
        "ln1_g": (d,), "ln1_b": (d,), "q_w": (d, d), "q_b": (d,), "k_w": (d, d),
        "v_w": (d, d), "v_b": (d,), "o_w": (d, d), "o_b": (d,), "ln2_g": (d,), "ln2_b": (d,),
        "fc1_w": (f, d), "fc1_b": (f,), "fc2_w": (d, f), "fc2_b": (d,),
    }
    for layer in range(g.n_layers):
        for name in LAYER_TENSORS:
            out.append((f"layers.{layer}.{name}", per_layer[name]))
    out += [("lnf_g", (d,)), ("lnf_b", (d,))]
    return out


def proj_shapes(g: Geometry) -> List[Tuple[str, Tuple[int, ...]]]:
    if not g.has_projector:
        return []
    return [("proj1_w", (g.proj_hidden, g.proj_in)), ("proj1_b", (g.proj_hidden,)),
            ("proj2_w", (g.proj_out, g.proj_hidden)), ("proj2_b", (g.proj_out,))]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _kind(name: str) -> str:
    base = name.rsplit(".", 1)[-1]
    if base.endswith("_g"):
        return "gamma"
    if base.endswith("_b"):
        return "beta" if base.startswith("ln") else "bias"
    return "weight"


def _draw(ss: np.random.SeedSequence, name: str, shape, init: str) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    z = rng.standard_normal(size=shape, dtype=np.float32)
    kind = _kind(name)
    base = name.rsplit(".", 1)[-1]
    if kind == "weight":
        std = SHARP_QK_STD if (init == "sharp" and base in ("q_w", "k_w")) else WEIGHT_STD
        return z * np.float32(std)
    if init == "paper" or init == "sharp":
        # N(0, 0.02) weights, zero biases, LayerNorm gamma = 1 and beta = 0.
        return np.ones(shape, np.float32) if kind == "gamma" else np.zeros(shape, np.float32)
    if init == "perturbed":
        # Nonzero biases, gamma and beta so that epilogue mistakes show.
        if kind == "gamma":
            return np.float32(1.0) + z * np.float32(WEIGHT_STD)
        return z * np.float32(WEIGHT_STD)
    raise ValueError(f"unknown init scheme {init!r}")


def make_weights(w: Workload) -> Dict[str, np.ndarray]:
    """All tensors of the workload as float32 arrays (bf16-exact for bf16)."""
    g = w.geom
    enc = weight_shapes(g)
    pj = proj_shapes(g)
    jobs = list(zip(enc, np.random.SeedSequence(w.weight_seed).spawn(len(enc))))
    jobs += list(zip(pj, np.random.SeedSequence(w.proj_seed).spawn(len(pj))))

    def one(job):
        (name, shape), ss = job
        x = _draw(ss, name, shape, w.init)
        return name, (round_to_bf16(x) if g.dtype == BF16 else x)

    # Each tensor owns its stream, so drawing them on several threads gives
    # the same values as drawing them in order.
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as pool:
        return dict(pool.map(one, jobs))


def make_lengths(w: Workload, n: int = None) -> np.ndarray:
    """Valid mel frames of clips 0..n-1 (default: the batch), int64; all F for
    fixed-length workloads. Clip i's length does not depend on n.

    Clip durations are uniform in [1 s, 30 s] at 100 frames per second
    ("Voxtral-Mini-3B-2507", Preprocessor: hop 160 at 16 kHz).
    """
    g = w.geom
    n = g.batch if n is None else n
    if not w.varlen:
        return np.full(n, g.n_frames, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.lengths_seed)))
    seconds = rng.uniform(1.0, 30.0, size=n)
    return np.clip(np.rint(100.0 * seconds), 100, g.n_frames).astype(np.int64)


def make_mel(w: Workload, clips=None) -> np.ndarray:
    """Mel features [len(clips), n_mel, F] float32; frames past a clip's length are 0."""
    g = w.geom
    clips = list(range(g.batch) if clips is None else clips)
    lengths = make_lengths(w, max(clips) + 1 if clips else 0)
    out = np.empty((len(clips), g.n_mel, g.n_frames), np.float32)
    for j, i in enumerate(clips):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.mel_seed, spawn_key=(int(i),))))
        x = rng.standard_normal(size=(g.n_mel, g.n_frames), dtype=np.float32)
        if w.mel_clip is not None:
            np.clip(x, -w.mel_clip, w.mel_clip, out=x)
        x[:, int(lengths[i]):] = 0.0
        out[j] = x
    if g.dtype == BF16:
        out = round_to_bf16(out)
    return out


def make_audio(seed: int, clips: int, n_samples: int = 480000, sample_rate: int = 16000) -> np.ndarray:
    """Seeded synthetic 16 kHz waveforms [clips, n_samples] float32 in [-1, 1].

    Speech-like stand-ins (no audio data is available): per clip a few
    harmonic tone stacks with drifting pitch and a syllable-rate amplitude
    envelope, plus low-level noise and short silent gaps, so the spectra
    have both peaks and an 80 dB-deep floor. Clip i draws stream (seed, i).
    """
    t = np.arange(n_samples, dtype=np.float64) / sample_rate
    out = np.empty((clips, n_samples), np.float32)
    for i in range(clips):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(int(i),))))
        x = np.zeros(n_samples)
        for _ in range(3):
            f0 = rng.uniform(90.0, 260.0)
            drift = rng.uniform(-0.3, 0.3) * np.sin(2 * np.pi * rng.uniform(0.1, 0.5) * t)
            phase = 2 * np.pi * np.cumsum(f0 * (1.0 + 0.1 * drift)) / sample_rate
            for h in range(1, 12):
                x += rng.uniform(0.2, 1.0) / h * np.sin(h * phase + rng.uniform(0, 2 * np.pi))
        env = 0.5 + 0.5 * np.sin(2 * np.pi * rng.uniform(2.0, 6.0) * t + rng.uniform(0, 2 * np.pi))
        x = x * env ** 2 + 0.02 * rng.standard_normal(n_samples)
        for _ in range(4):                        # silent gaps
            a = int(rng.integers(0, n_samples - 8000))
            x[a:a + int(rng.integers(1600, 8000))] *= 1e-4
        out[i] = (0.9 * x / np.abs(x).max()).astype(np.float32)
    return out


def make_mask(w: Workload, clips=None):
    """Key-padding mask uint8 [len(clips), T] (1 = valid), or None if all valid.

    A clip of n_f valid frames has ceil(n_f / 2) valid positions.
    """
    if not w.varlen:
        return None
    g = w.geom
    clips = list(range(g.batch) if clips is None else clips)
    lengths = make_lengths(w, max(clips) + 1 if clips else 0)
    t = np.arange(g.n_pos)
    valid = (lengths + 1) // 2
    return np.stack([(t < valid[i]).astype(np.uint8) for i in clips])
