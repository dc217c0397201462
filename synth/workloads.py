"""Geometries and named workloads of the Whisper-style audio encoder tower.

Geometry facts come from the model records on the pages:
  * Whisper-large encoder (d_model 1280, 32 layers, 20 heads, FFN 5120,
    128 mel bins, 1500 source positions): "Qwen2-Audio-7B-Instruct",
    section "(1) AUDIO ENCODER"; head_dim 64 with as many KV heads as query
    heads: "Voxtral-Mini-3B-2507", section "(1) AUDIO ENCODER".
  * 3000 feature frames per 30 s chunk: "Voxtral-Mini-3B-2507",
    "Preprocessor" (nb_max_frames, hop 160 at 16 kHz = 100 frames/s).
  * Whisper-medium encoder (d_model 1024, 24 layers, 16 heads, FFN 4096) and
    audio_pool_step 2: "MiniCPM-o-2_6", section "(2) AUDIO".
  * audio_chunk_length 1.0 next to the Whisper-medium encoder: "MiniCPM-o-2_6",
    section "(2) AUDIO" (the pages print the field without its semantics;
    the chunked attention workload takes it as 1 s = 50 positions per chunk).
  * 2-layer GELU projector into the 3072-wide LLM: "Voxtral-Mini-3B-2507",
    section "PROJECTOR".
  * Stacking 4 consecutive encoder positions into one 5120-wide projector
    input (50 -> 12.5 positions per second): Whisper features downsampled to
    12.5 Hz ("[WIP][TSS][Model] Kimi-Audio-7B", Purpose, Audio Tokenizer),
    kimia_adaptor_input_dim 5120 ("Kimi-Audio-7B-Instruct", (1) AUDIO).

A workload is named for what it is and fixes the seeds of every tensor.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Geometry:
    batch: int
    n_mel: int
    n_frames: int          # F = 2T mel frames per clip
    d_model: int
    n_layers: int
    n_heads: int
    d_ffn: int
    pool_step: int = 1     # 1 (none) or 2 (average pool of position pairs)
    proj_hidden: int = 0   # 0 = no projector
    proj_out: int = 0
    dtype: str = BF16      # weights, mel and activations
    out_dtype: str = F32
    ln_eps: float = 1e-5
    stack: int = 1         # positions concatenated into one projector input row (1 or 4)
    attn_chunk: int = 0    # positions per attention chunk (0: every position sees every position)
    attn_chunk_mode: int = 0   # with attn_chunk: 1 chunk-causal, 2 block-diagonal

    @property
    def n_pos(self) -> int:
        """Positions T of the input contract: a clip of F = 2T frames."""
        return self.n_frames // 2

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def has_projector(self) -> bool:
        return self.proj_hidden > 0

    @property
    def t_out(self) -> int:
        return self.n_pos // self.pool_step // self.stack

    @property
    def proj_in(self) -> int:
        """Width of a projector input row: stack consecutive positions."""
        return self.stack * self.d_model

    @property
    def d_out(self) -> int:
        return self.proj_out if self.has_projector else self.d_model

    def replace(self, **kw) -> "Geometry":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    weight_seed: int = 0
    proj_seed: int = 2
    mel_seed: int = 1
    lengths_seed: Optional[int] = None   # set: variable-length clips with a key mask
    mel_clip: Optional[float] = None     # clip mel values to [-c, c]
    init: str = "paper"                  # "paper": N(0,0.02) weights, zero biases, unit gamma
    description: str = ""

    @property
    def varlen(self) -> bool:
        return self.lengths_seed is not None

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WHISPER_LARGE = dict(n_mel=128, n_frames=3000, d_model=1280, n_layers=32, n_heads=20, d_ffn=5120)
WHISPER_MEDIUM = dict(n_mel=80, n_frames=3000, d_model=1024, n_layers=24, n_heads=16, d_ffn=4096)

WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(
            "tiny_fp32_b1",
            Geometry(batch=1, n_mel=80, n_frames=200, d_model=256, n_layers=2, n_heads=4,
                     d_ffn=1024, dtype=F32, out_dtype=F32),
            mel_clip=4.0,
            description="tiny encoder, fp32, 200 frames -> 100 positions, 2 blocks of d 256",
        ),
        Workload(
            "whisper_medium_pool2_b1",
            Geometry(batch=1, pool_step=2, **WHISPER_MEDIUM),
            description="Whisper-medium encoder, bf16, batch 1, average pool step 2 -> 750 tokens",
        ),
        Workload(
            "whisper_medium_pool2_chunk1s_b16",
            Geometry(batch=16, pool_step=2, attn_chunk=50, attn_chunk_mode=1, **WHISPER_MEDIUM),
            description="Whisper-medium encoder, bf16, batch 16, pool step 2, attention in 1 s chunks "
                        "(50 positions), each chunk seeing itself and the chunks before it",
        ),
        Workload(
            "whisper_large_b1",
            Geometry(batch=1, **WHISPER_LARGE),
            description="Whisper-large encoder, bf16, batch 1",
        ),
        Workload(
            "whisper_large_proj_b16",
            Geometry(batch=16, proj_hidden=3072, proj_out=3072, **WHISPER_LARGE),
            description="Whisper-large encoder, bf16, batch 16, GELU projector 1280->3072->3072",
        ),
        Workload(
            "whisper_large_stack4_proj_b16",
            Geometry(batch=16, proj_hidden=3072, proj_out=3072, stack=4, **WHISPER_LARGE),
            description="Whisper-large encoder, bf16, batch 16, 4 positions stacked (12.5 Hz) into a "
                        "GELU projector 5120->3072->3072",
        ),
        Workload(
            "whisper_large_varlen_b32",
            Geometry(batch=32, **WHISPER_LARGE),
            lengths_seed=3,
            description="Whisper-large encoder, bf16, 32 clips of 1-30 s padded to 3000 frames, key mask",
        ),
    ]
}

# The workload the throughput figure is quoted on (fits one GPU).
HEADLINE = "whisper_large_proj_b16"


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
