"""Seeded synthetic inputs for the KDA chunked forward.

This package draws random inputs and rounds them to bfloat16. It holds none of
the method's arithmetic: both the CPU oracle side (tests) and the GPU side
(tests, bench, smoke) take their inputs from here, and nothing else is shared.
"""
from .inputs import CONFIGS, make_inputs, make_config_inputs, round_to_bf16, bf16_bits  # noqa: F401
