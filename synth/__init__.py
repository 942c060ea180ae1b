"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and the benchmark.

This package holds shapes, seeds and random draws only. It contains none of the attention
arithmetic (no normalisation, no sigmoid, no logits), so the oracle and the HIP path can both
take their inputs from it without sharing any of the method's code.
"""
from .inputs import CONFIGS, Workload, make_inputs, round_to_dtype, bf16_round  # noqa: F401
