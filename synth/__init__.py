"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package holds shapes and random draws only: none of the quantisation,
packing, permutation or product arithmetic lives here.
"""
from .inputs import (  # noqa: F401
    LinearSpec, StackSpec, CONFIGS, SPACES, stack_spec, small_stack_spec,
    weight, decode_input, profile, planted_set, config1_inputs,
    planted_count, generate_parallel, vocab_size, embedding, token_ids,
)
