"""Seeded synthetic KV workloads shared by the tests, the smoke check and the bench.

This module draws random numbers and rounds them to bf16 inputs; it holds none of the codec's
arithmetic, and both the HIP path and the CPU oracle receive the same arrays from it.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    bf16_bits,
    bf16_to_f32,
    c1_tensors,
    c2_tensors,
    c3_chain_inputs,
    c4_tensors,
    c4_residual_target,
    c5_tensors,
    c5_residual_targets,
    tiny_tensor,
    normal_kv,
)
