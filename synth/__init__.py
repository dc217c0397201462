"""Seeded synthetic workloads for the audio encoder tower.

This package is shared by the CPU oracle, the tests and the benchmark. It
holds geometry tables and seeded random generators only: none of the
encoder's arithmetic lives here.
"""
from .workloads import Geometry, Workload, WORKLOADS, get_workload  # noqa: F401
from .inputs import (  # noqa: F401
    weight_shapes, make_weights, make_mel, make_lengths, make_mask, make_audio,
    to_bf16_bits, bf16_bits_to_f32, round_to_bf16,
)
