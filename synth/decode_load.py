"""A synthetic LLM-decode load that shares the GPU with the encoder.

Serving stacks run the audio encoder on a stream of its own, beside the
language model's decode steps (TRT-LLM's "Multimodal Encoder Side Stream",
listed under (1) SERVICEABILITY JOIN of the "Kimi-Audio-7B-Instruct" and
"Qwen2-Audio-7B-Instruct" records). To measure how well the two overlap, this
module stands in for the decode side: one step multiplies a small batch of
token rows through every layer's weights, which is what makes decode
HBM-bound (each step streams all weights once).

Layer shapes follow the LLM printed in the "Kimi-Audio-7B-Instruct" record,
section (2) LLM: 28 layers, hidden 3584, 28 query heads and 4 KV heads of
128 (a fused QKV weight of 3584 + 2 * 512 rows), intermediate 18944 (a fused
gate/up weight of 2 * 18944 rows). Attention over the KV cache and the norms
are left out: at decode they move little data next to the weights.

This is a load generator, not part of the encoder: it runs plain torch
products (hipBLASLt) on whatever stream is current. Weights
are seeded random values scaled by 1/sqrt(fan-in), so activations stay O(1).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    layers: int = 28
    hidden: int = 3584
    kv_dim: int = 512          # 4 KV heads x 128
    inter: int = 18944
    tokens: int = 16           # decode rows per step

    def weight_bytes(self) -> int:
        """bf16 bytes one step streams (every weight once)."""
        h = self.hidden
        per_layer = (h + 2 * self.kv_dim) * h + h * h + 2 * self.inter * h + h * self.inter
        return 2 * self.layers * per_layer


KIMI_AUDIO_LLM = DecodeShape()


class DecodeLoad:
    """Device weights of `shape` and a step() that enqueues one decode step on
    torch's current stream."""

    def __init__(self, shape: DecodeShape = KIMI_AUDIO_LLM, seed: int = 11, device="cuda"):
        import torch
        self.shape = shape
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        h, kv, it = shape.hidden, shape.kv_dim, shape.inter

        def w(rows, cols):
            t = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
            return (t * cols ** -0.5).to(torch.bfloat16)

        self.layers = [(w(h + 2 * kv, h), w(h, h), w(2 * it, h), w(h, it)) for _ in range(shape.layers)]
        self.x0 = torch.randn(shape.tokens, h, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)

    def step(self, x=None):
        """One decode step over all layers; returns the final rows [tokens, hidden].

        Four products per layer and nothing else, so that the host enqueues
        a step faster than the GPU streams its weights: the attention output
        is stood in for by the query columns of the QKV product and the
        gated activation by the gate half of the gate/up product (strided
        views, no copies)."""
        import torch.nn.functional as F
        x = self.x0 if x is None else x
        h, it = self.shape.hidden, self.shape.inter
        for wqkv, wo, wgu, wd in self.layers:
            qkv = F.linear(x, wqkv)
            x = F.linear(qkv[:, :h], wo)
            gu = F.linear(x, wgu)
            x = F.linear(gu[:, :it], wd)
        return x
