"""Seeded synthetic inputs for the FAST-AR attention step.

This package only draws random inputs (centroid-clustered keys that drift from
frame to frame, noisy queries, prompt tokens, hyperplanes) and rounds them to
the storage precision. It contains none of the method's arithmetic: no hashing,
no attention, no cache policy. Both the CPU oracle and the HIP path consume the
exact same bytes produced here.
"""
from .gen import (CONFIGS, WorkloadConfig, Step, make_step, rollout_chunks, commit_case, group_sizes,
                  table_planes, codebook_from_keys,
                  bf16_round, bf16_bits_to_f32, f32_to_bf16_bits)

__all__ = ["CONFIGS", "WorkloadConfig", "Step", "make_step", "rollout_chunks", "commit_case", "group_sizes",
           "table_planes", "codebook_from_keys",
           "bf16_round", "bf16_bits_to_f32", "f32_to_bf16_bits"]
