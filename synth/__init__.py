"""Seeded synthetic inputs for one verify round of one-pass block drafting.

This package only draws random numbers and lays them out. It holds none of the
method's arithmetic (no softmax of the draft head, no tree selection, no
attention, no head statistics), so both the CPU oracle and the HIP path can
consume its arrays without sharing any computation.
"""
from .gen import (  # noqa: F401
    RoundConfig,
    CONFIGS,
    bf16_bits,
    bf16_bits_to_f32,
    gen_round,
    make_config,
)
