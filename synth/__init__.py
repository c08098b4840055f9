"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package holds no arithmetic of the quantization method: it only draws
numbers (SplitMix64 -> uniform -> Box-Muller normal / Student-t) and shapes
them into the activation and latent-weight tensors of the workloads.
"""
from .generators import (  # noqa: F401
    splitmix64, uniform01, normal, student_t3, to_bf16_bits, bf16_bits_to_f32,
    activations_bf16, latent_weights, outlier_channels, rope_tables, WORKLOADS, workload_inputs,
)
