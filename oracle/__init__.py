"""CPU oracle of the Whisper-style audio encoder tower (test infrastructure).

This package is a plain, slow, fp64 NumPy statement of what the encoder
computes. It exists to check the GPU library, and only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. The product
path never calls it, and it shares no code with the HIP kernels or their
host runtime; the two meet only through the seeded inputs of ``synth``.
"""
from .encoder import (  # noqa: F401
    gelu, layer_norm, conv1d_k3, sinusoids, linear, attention, attention_core, block, blocks, stem,
    final, encode_clip, encode, param_count, param_shapes, flops, chunk_allowed, attended_pairs,
    CHUNK_CAUSAL, CHUNK_BLOCK,
)
