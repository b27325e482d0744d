"""Seeded synthetic inputs for the Q4 expert gate/up path.

This package only draws random numbers and lays bytes out in an expert slot.
It holds none of the method's arithmetic (no dequantisation, no dot products,
no rounding of results), so both the CPU oracle and the HIP path can use it
without sharing any of the computation under test.
"""

from .generators import (  # noqa: F401
    OFFSET_ABSENT,
    SlotLayout,
    contiguous_layout,
    expert_layout,
    pack_nibbles,
    fill_slot,
    write_slot,
    bf16_normal,
    add_outliers,
    f32_normal,
    add_outliers_f32,
    top_k_routing,
    Config,
    CONFIGS,
    make_config,
    sha256_hex,
)
