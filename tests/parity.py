"""Helpers of the GPU parity tests: tolerance checks, device copies of the
seeded inputs, and oracle outputs (computed, or read back from the cache that
tests/golden/make_oracle_cache.py writes by calling only the oracle)."""
from __future__ import annotations

import hashlib
import inspect
import json
import os
from typing import Dict, Optional, Sequence

import numpy as np

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CACHE_DIR = os.path.join(ROOT, "tests", ".oracle_cache")

# Tolerances of the GPU path against the fp64 oracle.
BF16_MAX_ABS = 3e-2
BF16_MIN_ROW_COS = 0.999
F32_MAX_REL = 1e-4


def metrics(got: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    """max-abs, min row cosine (rows = last axis) and normwise max-rel."""
    g = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    diff = np.abs(g - r)
    num = (g * r).sum(1)
    den = np.linalg.norm(g, axis=1) * np.linalg.norm(r, axis=1)
    cos = np.where(den > 0, num / np.maximum(den, 1e-300), 1.0)
    return {"max_abs": float(diff.max()), "min_row_cos": float(cos.min()),
            "max_rel": float(diff.max() / max(np.abs(r).max(), 1e-300)),
            "finite": bool(np.isfinite(g).all())}


def assert_bf16_parity(got, ref, what=""):
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_abs"] <= BF16_MAX_ABS and m["min_row_cos"] >= BF16_MIN_ROW_COS, f"{what}: {m}"
    return m


def assert_f32_parity(got, ref, what=""):
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_rel"] <= F32_MAX_REL, f"{what}: {m}"
    return m


# ---------------------------------------------------------------------------
# Oracle outputs, cached per (workload, clip, rows) and keyed on the oracle's source.
# ---------------------------------------------------------------------------

def _digest():
    """A fast digest over whole byte buffers (xxh3 when the xxhash package is
    present, else SHA-256)."""
    try:
        import xxhash
        return xxhash.xxh3_128()
    except ImportError:
        return hashlib.sha256()


def _fingerprint(W: dict, mel: np.ndarray, mask) -> str:
    """Digest of every byte the oracle reads: all weight tensors in full, the
    mel input and the mask."""
    h = _digest()
    for name in sorted(W):
        h.update(name.encode() + str(W[name].shape).encode())
        h.update(np.ascontiguousarray(W[name], np.float32).data)
    h.update(np.ascontiguousarray(mel, np.float32).data)
    if mask is not None:
        h.update(np.ascontiguousarray(mask).data)
    return h.hexdigest()


def _sources_digest() -> str:
    """The oracle's source and the seeded input generators' source."""
    h = hashlib.sha256()
    for mod in (oracle.encoder, synth.inputs, synth.workloads):
        h.update(inspect.getsource(mod).encode())
    return h.hexdigest()


def _key(w: synth.Workload, clip: int, W: dict, mel: np.ndarray, mask) -> str:
    spec = json.dumps({"geom": repr(w.geom), "clip": clip, "data": _fingerprint(W, mel, mask),
                       "sources": _sources_digest()}, sort_keys=True)
    return hashlib.sha256(spec.encode()).hexdigest()[:24]


def sample_rows(n: int, every: int) -> np.ndarray:
    rows = set(range(0, n, every)) | {0, 1, n - 2, n - 1}
    return np.array(sorted(r for r in rows if 0 <= r < n))


def oracle_clip(w: synth.Workload, clip: int, W: Optional[dict] = None, every: int = 1,
                use_cache: bool = True) -> Dict[str, np.ndarray]:
    """Oracle output of one clip: {"rows": indices, "out": [len(rows), D_out]} (fp64).

    The clip runs alone (clips are independent) with its own mask row. The
    cache key covers the geometry, a digest of every weight and input byte,
    and the source of the oracle and of the input generators, so a stale
    entry is never read.
    """
    if W is None:
        W = synth.make_weights(w)
    mel = synth.make_mel(w, clips=[clip])[0]
    mask = synth.make_mask(w, clips=[clip])
    path = os.path.join(CACHE_DIR, f"{w.name}-{_key(w, clip, W, mel, mask)}-e{every}.npz")
    if use_cache and os.path.exists(path):
        with np.load(path) as z:
            return {"rows": z["rows"], "out": z["out"].astype(np.float64)}
    out = oracle.encode_clip(w.geom, W, mel, None if mask is None else mask[0])
    rows = sample_rows(out.shape[0], every)
    res = {"rows": rows, "out": out[rows]}
    if use_cache:
        os.makedirs(CACHE_DIR, exist_ok=True)
        np.savez(path + ".tmp.npz", rows=rows, out=res["out"].astype(np.float32))
        os.replace(path + ".tmp.npz", path)
        res["out"] = res["out"].astype(np.float32).astype(np.float64)
    return res


# Full-size workloads: which clips and rows the parity tests compare.
FULL_SIZE_SAMPLES = {
    "tiny_fp32_b1": dict(clips=[0], every=1),
    "whisper_medium_pool2_b1": dict(clips=[0], every=1),
    "whisper_large_b1": dict(clips=[0], every=1),
    "whisper_large_proj_b16": dict(clips=[0, 7, 15], every=5),
    "whisper_large_stack4_proj_b16": dict(clips=[0, 15], every=3),
    "whisper_large_varlen_b32": dict(clips=None, every=5),   # shortest, longest and one in between
    "whisper_medium_pool2_chunk1s_b16": dict(clips=[0, 15], every=3),
}


# Further oracle outputs the GPU tests read (whole clips): the distinct mels of
# the last two clips of the largest-batch test.
EXTRA_CLIPS = {"whisper_large_b1": [1, 2]}


def varlen_sample_clips(w: synth.Workload) -> Sequence[int]:
    lengths = synth.make_lengths(w)
    order = np.argsort(lengths, kind="stable")
    return sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})


def full_size_clips(w: synth.Workload) -> Sequence[int]:
    spec = FULL_SIZE_SAMPLES[w.name]
    return varlen_sample_clips(w) if spec["clips"] is None else spec["clips"]
